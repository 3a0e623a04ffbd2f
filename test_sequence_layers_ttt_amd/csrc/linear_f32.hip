// TTT-Linear forward scan with fp32 I/O on the fp32 matrix cores: d in {16, 32,
// 64, 128}, any chunk length, the inclusive read.
//
// Method: PaperTrace "5 · TestingTime 训练与长上下文" §1.1 and §2.3 (every
// gradient of a chunk at the chunk-start state W_c; token t reads the chunk's
// updates up to and including its own), in the dual form of diosapp
// "Test-Time Training (TTT) guide" §3, walked in 16-token sub-tiles with tokens
// as columns:
//   E = W_c K - V,  Z = M Q - E diag(eta) (U o K^T Q),  M <- M - E diag(eta) K^T,
// U the causal mask (s <= t), M the running state (= W_c at a chunk start, and
// W_{c+1} = M at the chunk end).
//
// Row i of Z and of the state depends only on row i of W0 and feature i of V, so
// the unit is one (batch, head) and one block of 16 state rows, and one wave
// owns it: rows r0 + c (c = lane % 16) of W_c and M in registers, all columns.
// Every product is a 16 x 16 tile product on v_mfma_f32_16x16x4_f32 (exact fp32
// products, fp32 sums), in the transposed orientation that keeps the state's
// rows in the lanes (see mfma_f32.h):
//   E^T = K W_c^T - V^T,  P^T = Q M^T,  S = K Q^T,
//   Z^T = P^T - S^T (E diag(eta))^T,  M^T <- M^T - K^T (E diag(eta))^T,
// so that E, P and Z all sit as "lane = state row r0 + c, slots = tokens
// 4g .. 4g+3" and the update lands in the layout the next products read.  The
// next sub-tile's K, Q, V and eta are loaded as raw words while the current one
// is computed; Z goes out through range-checked buffer stores.  The units of one
// head are placed on one XCD, sharing its L2 for K and Q.
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "mfma_f32.h"

namespace ttt {
namespace {

constexpr int kSub = 16;
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a gfx9 buffer resource: raw 32-bit data

// One sub-tile's inputs as loaded by lane t: D/4 consecutive features of K and Q
// of token t / 4, 4 of V (the wave's 16 state rows) of the same token, eta of
// token t % 16.
template <int D>
struct F32Tile {
    RawRow<float, D / 4> k, q;
    RawRow<float, 4> v;
    float eta;
};

template <int D>
struct F32Lds {
    static constexpr int S = D + 4;   // row stride of the token x feature tiles
    float K[kSub * S];
    float Q[kSub * S];
    float V[kSub * 20];               // [token][state row - r0]
    float eta[kSub];
};

template <int D, bool ETA>
__global__ __launch_bounds__(64) void linear_f32_kernel(
    const float* __restrict__ K, const float* __restrict__ Q, const float* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar, const float* W0, float* __restrict__ Z,
    float* W_out, int BH, int T, int chunk)
{
    constexpr int NB = D / 16, S = F32Lds<D>::S, EP = D / 4;
    __shared__ __align__(16) F32Lds<D> L;

    const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
    int slice, rb;
    xcd_unit_part(blockIdx.x, NB, slice, rb);
    if (slice >= BH) return;
    const int r0 = 16 * rb;   // this wave's state rows
    const size_t tok0 = (size_t)slice * T;
    const int fs = lane >> 2, fq = lane & 3;   // staged token, quarter of its features

    // state rows r0 + c, columns 16b + 4g .. 16b + 4g + 3 of block b (RL form)
    f32x4 Wc[NB], M[NB];
    {
        const float* w = W0 + ((size_t)slice * D + r0 + c) * D + 4 * g;
#pragma unroll
        for (int b = 0; b < NB; ++b) Wc[b] = M[b] = *reinterpret_cast<const f32x4*>(w + 16 * b);
    }

    const int nsub = (chunk + kSub - 1) / kSub;   // sub-tiles of a full chunk
    const int last = (T - 1) / chunk * nsub + ((T - 1) % chunk) / kSub;
    // sub-tile j: position si in its chunk, tokens [t0, t0 + len)
    auto span = [&](int j, int& si, int& t0, int& len) {
        const int ch = j / nsub;
        si = j - ch * nsub;
        t0 = ch * chunk + si * kSub;
        len = min(kSub, min(ch * chunk + chunk, T) - t0);
    };
    // every load reads a token of the sub-tile (tokens past its end re-read the
    // last one), so every path issues the same loads
    auto fetch = [&](F32Tile<D>& f, int j) {
        int si, t0, len;
        span(j, si, t0, len);
        const size_t row = (tok0 + t0 + min(fs, len - 1)) * D;
        f.k.load(K + row + fq * EP);
        f.q.load(Q + row + fq * EP);
        f.v.load(V + row + r0 + 4 * fq);
        if constexpr (ETA) f.eta = eta[tok0 + t0 + min(c, len - 1)];
        else f.eta = eta_scalar;
    };
    // Tokens past the sub-tile's end stage the re-read last token as it is: every
    // contribution of such a token is scaled by its masked E diag(eta) below (a
    // finite value times zero), and its own outputs are never stored.  (A select
    // here would be hoisted onto the freshly loaded registers and wait for them.)
    auto put = [&](const F32Tile<D>& f) {
#pragma unroll
        for (int i = 0; i < EP; i += 4) {
            *reinterpret_cast<f32x4*>(L.K + fs * S + fq * EP + i) =
                f32x4{f.k.at(i), f.k.at(i + 1), f.k.at(i + 2), f.k.at(i + 3)};
            *reinterpret_cast<f32x4*>(L.Q + fs * S + fq * EP + i) =
                f32x4{f.q.at(i), f.q.at(i + 1), f.q.at(i + 2), f.q.at(i + 3)};
        }
        *reinterpret_cast<f32x4*>(L.V + fs * 20 + 4 * fq) =
            f32x4{f.v.at(0), f.v.at(1), f.v.at(2), f.v.at(3)};
        if (lane < kSub) L.eta[lane] = f.eta;
    };

    // two prefetch slots used alternately at compile-time positions
    F32Tile<D> bufs[2];
    auto step = [&](int j, auto slot) {
        auto& cur = bufs[decltype(slot)::value];
        auto& nxt = bufs[decltype(slot)::value ^ 1];
        int si, t0, len;
        span(j, si, t0, len);
        __syncthreads();   // the previous sub-tile's tiles are consumed
        put(cur);
        __syncthreads();
        if (j < last) fetch(nxt, j + 1);
        // keep the loads here: sunk below this sub-tile's stores, they would make
        // the next staging wait for those stores too
        __builtin_amdgcn_sched_barrier(0);
        // E^T = K W_c^T - V^T, P^T = Q M^T, S = K Q^T, over the features
        f32x4 E = -cl<20>(L.V, 0, lane), P = {0.f, 0.f, 0.f, 0.f}, Sc = P;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const f32x4 kb = rl<S>(L.K, 16 * b, lane), qb = rl<S>(L.Q, 16 * b, lane);
            E = mm16(kb, Wc[b], E);
            P = mm16(qb, M[b], P);
            Sc = mm16(kb, qb, Sc);
        }
        // causal scores: writer s = 4g + v, reader t = c
        f32x4 Sm;
#pragma unroll
        for (int v = 0; v < 4; ++v) Sm[v] = (4 * g + v <= c) ? Sc[v] : 0.f;
        // E diag(eta); tokens past the sub-tile's end contribute nothing
        const f32x4 et = *reinterpret_cast<const f32x4*>(L.eta + 4 * g);
        f32x4 Ee;
#pragma unroll
        for (int v = 0; v < 4; ++v) Ee[v] = (4 * g + v < len) ? E[v] * et[v] : 0.f;
        // Z^T = P^T - S^T (E eta)^T: A = RL(S^T) = CL(S), B = CL((E eta)^T) = Ee
        const f32x4 Zt = P - mm16(Sm, Ee, f32x4{0.f, 0.f, 0.f, 0.f});
        // Z[t0 + 4g + v][r0 + c]; tokens past the sub-tile's end fall outside the range
        {
            const auto rz = __builtin_amdgcn_make_buffer_rsrc(Z + (tok0 + t0) * D, 0,
                                                             (int)(len * D * sizeof(float)),
                                                             kBufferFlags);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(Zt[v]), rz,
                                                      ((4 * g + v) * D + r0 + c) * 4, 0, 0);
        }
        // M^T -= K^T (E eta)^T per column block: A = RL(K^T_b) = CL(K_b), B = -Ee
        const f32x4 nEe = -Ee;
#pragma unroll
        for (int b = 0; b < NB; ++b) M[b] = mm16(cl<S>(L.K, 16 * b, lane), nEe, M[b]);
        // chunk end: the running state becomes the next chunk-start state
        if (si == nsub - 1 || j == last) {
#pragma unroll
            for (int b = 0; b < NB; ++b) Wc[b] = M[b];
        }
    };
    const std::integral_constant<int, 0> slot0;
    const std::integral_constant<int, 1> slot1;
    // the first sub-tile runs before the loop, so that the loop is entered, as it
    // is re-entered, with a sub-tile's stores behind the prefetched loads (the
    // waits at the loop head then cover the loads only)
    fetch(bufs[0], 0);
    step(0, slot0);
    {
        int j = 1;
        for (; j + 1 <= last; j += 2) {
            step(j, slot1);
            step(j + 1, slot0);
        }
        if (j == last) step(j, slot1);
    }

    float* w = W_out + ((size_t)slice * D + r0 + c) * D + 4 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(w + 16 * b) = M[b];
}

template <int D>
void launch_d(const LinearArgs& a, hipStream_t s)
{
    // (batch*head, 16-row block) units, the blocks of one head on one XCD
    const dim3 grid((unsigned)(((a.BH + 7) / 8) * 8 * (D / 16))), block(64);
    const float* K = static_cast<const float*>(a.K);
    const float* Q = static_cast<const float*>(a.Q);
    const float* V = static_cast<const float*>(a.V);
    float* Z = static_cast<float*>(a.Z);
    if (a.eta)
        hipLaunchKernelGGL((linear_f32_kernel<D, true>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W0, Z, a.W_out, a.BH, a.T, a.chunk);
    else
        hipLaunchKernelGGL((linear_f32_kernel<D, false>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W0, Z, a.W_out, a.BH, a.T, a.chunk);
}

}  // namespace

bool linear_f32_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t s)
{
    switch (a.d) {
    case 16: launch_d<16>(a, s); break;
    case 32: launch_d<32>(a, s); break;
    case 64: launch_d<64>(a, s); break;
    case 128: launch_d<128>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ttt
