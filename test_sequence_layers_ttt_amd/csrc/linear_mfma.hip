// TTT-Linear forward scan on gfx950 matrix cores (bf16 operands, fp32 state).
//
// Method: PaperTrace "5 · TestingTime 训练与长上下文" §1.1/§2.3 (chunked update,
// gradient of 1/2||W k - v||^2 at the chunk-start state, inclusive read), in the
// dual form of diosapp "Test-Time Training (TTT) guide" §3.  For a 16-token
// sub-tile with tokens as columns:
//     E = W_c K - V                 (gradient factor, at the chunk-start state)
//     Z = M Q - E diag(eta) triu(K^T Q)
//     M = M - E diag(eta) K^T       (running state; W_{c+1} = M at chunk end)
// For chunk <= 16 a sub-tile is one chunk (W_c = M); for a chunk that is a
// multiple of 16, E keeps using the frozen chunk-start W_c while M runs.
//
// Work split.  Row i of Z and of the state depends only on row i of W0 and
// feature i of V (and on all of K, Q, eta), so each wave owns 16 output rows of
// one (batch, head) and never talks to another wave.  The d/16 waves of a head
// are placed on one XCD so that they share that XCD's L2 for K and Q.
//
// Register dataflow (one wave; see mfma_common.h for the MFMA layouts).
//   M      : d/16 fp32 C/D tiles; tile jb, lane (o, g), value i holds
//            W[o][pi(jb, 4g+i)] with pi(2m, 4g+i) = 32m+8g+i and
//            pi(2m+1, 4g+i) = 32m+8g+4+i, so that the bf16 x32-operand of step
//            m is (tile 2m, tile 2m+1) packed, and K/Q rows load as 16 bytes.
//   E^T    = K^T W^T - V^T      : A = K rows (lane = token), B = W rows; C from
//            -V^T, which an identity product moves into C/D layout.
//   F      = -diag(eta) E^T in bf16 (C/D layout = B operand over tokens).
//   M_jb  += Kt_jb F            : Kt_jb = K tile transposed by an identity
//            product (lane = input feature, slots = tokens).
//   S^T    = K^T Q masked s<=t  : C/D layout = B operand over tokens.
//   Z^T    = W Q^T + F^T... :  A = W rows, B = Q rows, then A = F read as
//            (E diag(-eta)) rows, B = S^T; lane (t, g) ends with Z[t][4g..4g+3].
// No LDS, no barriers, no atomics.
#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int kStep = 16;

template <int D>
struct Tile {
    u32x4 k[D / 32];   // K row (lane = token), 16-byte pieces at 32m + 8g
    u32x4 q[D / 32];   // Q row, same pieces
    u32x2 v;           // V[token][out0 + 4g .. +3]
    f32x4 eta;         // eta of tokens 4g .. 4g+3 (C/D rows)
    int n;             // valid tokens (0 = past the end)
};

template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ Q,
                                          const uint16_t* __restrict__ V,
                                          const float* __restrict__ eta, float eta_scalar,
                                          size_t tok0, int s0, int n, int out0, int lane)
{
    const int c = lane & 15, g = lane >> 4;
    t.n = n;
    const bool live = c < n;
    const size_t row = (tok0 + s0 + (live ? c : 0)) * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
        u32x4 kk = *(const u32x4*)(K + row + 32 * m + 8 * g);
        u32x4 qq = *(const u32x4*)(Q + row + 32 * m + 8 * g);
        t.k[m] = live ? kk : u32x4{0, 0, 0, 0};
        t.q[m] = live ? qq : u32x4{0, 0, 0, 0};
    }
    u32x2 vv = *(const u32x2*)(V + row + out0 + 4 * g);
    t.v = live ? vv : u32x2{0, 0};
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = 4 * g + i;
        float x = eta ? eta[tok0 + s0 + (s < n ? s : 0)] : eta_scalar;
        e[i] = s < n ? x : 0.f;
    }
    t.eta = f32x4{e[0], e[1], e[2], e[3]};
}

template <int D, int PF>
__global__ __launch_bounds__(64) void linear_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, int BH, int T, int chunk)
{
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    const int lane = threadIdx.x;
    const int c = lane & 15, g = lane >> 4;
    int slice, ob;
    xcd_unit_part(blockIdx.x, NB, slice, ob);
    if (slice >= BH) return;
    const int out0 = ob * 16;
    const size_t tok0 = (size_t)slice * T;

    // state rows out0 + c, columns pi(jb, 4g + i)
    f32x4 M[NB];
    {
        const float* w = W0 + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[2 * m] = *(const f32x4*)(w + 32 * m + 8 * g);
            M[2 * m + 1] = *(const f32x4*)(w + 32 * m + 8 * g + 4);
        }
    }
    const u32x2 I16 = identity_b16(lane);

    const int step = chunk < kStep ? chunk : kStep;
    const int ntiles = (T + step - 1) / step;

    Tile<D> buf[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int s0 = p * step;
        const int n = s0 < T ? min(step, T - s0) : 0;
        load_tile<D>(buf[p], K, Q, V, eta, eta_scalar, tok0, n > 0 ? s0 : 0, n, out0, lane);
    }

    u32x4 Wc[NM];   // bf16 chunk-start state (operand of E)
    for (int tau0 = 0; tau0 < ntiles; tau0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int tau = tau0 + p;
            if (tau >= ntiles) break;
            Tile<D> cur = buf[p];
            {
                const int s0 = (tau + PF) * step;
                const int n = s0 < T ? min(step, T - s0) : 0;
                load_tile<D>(buf[p], K, Q, V, eta, eta_scalar, tok0, n > 0 ? s0 : 0, n, out0,
                             lane);
            }
            const int s0 = tau * step;
            // running state in bf16 (operand of W Q, and of E at a chunk start)
            u32x4 Mf[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
            if (s0 % chunk == 0) {
#pragma unroll
                for (int m = 0; m < NM; ++m) Wc[m] = Mf[m];
            }
            // E^T = K^T W_c^T - V^T
            u32x2 vneg = cur.v ^ u32x2{0x80008000u, 0x80008000u};
            f32x4 Et = mfma16(vneg, I16, f32x4{0, 0, 0, 0});
#pragma unroll
            for (int m = 0; m < NM; ++m) Et = mfma32(cur.k[m], Wc[m], Et);
            // F = -diag(eta) E^T  (bf16)
            const u32x2 F = pack_bf16x4(-cur.eta * Et);
            // S^T = K^T Q with the inclusive causal mask s <= t
            f32x4 St = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) St = mfma32(cur.k[m], cur.q[m], St);
            f32x4 Sm;
            Sm.x = (4 * g + 0 <= c) ? St.x : 0.f;
            Sm.y = (4 * g + 1 <= c) ? St.y : 0.f;
            Sm.z = (4 * g + 2 <= c) ? St.z : 0.f;
            Sm.w = (4 * g + 3 <= c) ? St.w : 0.f;
            const u32x2 Sb = pack_bf16x4(Sm);
            // Z^T = M Q^T - (E diag(eta)) S
            f32x4 Zt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Zt = mfma32(Mf[m], cur.q[m], Zt);
            Zt = mfma16(F, Sb, Zt);
            if (c < cur.n) {
                u32x2 zb = pack_bf16x4(Zt);
                *(u32x2*)(Z + (tok0 + s0 + c) * D + out0 + 4 * g) = zb;
            }
            // M += K F  (tile by tile; K transposed by the identity product)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                f32x4 t0 = mfma16(lo_half(cur.k[m]), I16, f32x4{0, 0, 0, 0});
                f32x4 t1 = mfma16(hi_half(cur.k[m]), I16, f32x4{0, 0, 0, 0});
                M[2 * m] = mfma16(pack_bf16x4(t0), F, M[2 * m]);
                M[2 * m + 1] = mfma16(pack_bf16x4(t1), F, M[2 * m + 1]);
            }
        }
    }

    float* w = W_out + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        *(f32x4*)(w + 32 * m + 8 * g) = M[2 * m];
        *(f32x4*)(w + 32 * m + 8 * g + 4) = M[2 * m + 1];
    }
}

template <int D>
hipError_t launch_d(const LinearArgs& a, hipStream_t s)
{
    constexpr int PF = 4;
    const int units = (a.BH + 7) / 8 * 8;
    dim3 grid((unsigned)(units * (D / 16))), block(64);
    hipLaunchKernelGGL((linear_mfma_kernel<D, PF>), grid, block, 0, s, (const uint16_t*)a.K,
                       (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta, a.eta_scalar, a.W0,
                       (uint16_t*)a.Z, a.W_out, a.BH, a.T, a.chunk);
    return hipGetLastError();
}

}  // namespace

bool linear_mfma_supported(int d, int chunk, int bf16)
{
    return bf16 && (d == 32 || d == 64 || d == 128) && (chunk <= kStep || chunk % kStep == 0);
}

hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s)
{
    switch (a.d) {
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ttt
