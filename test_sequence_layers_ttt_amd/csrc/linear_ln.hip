// TTT-Linear with the inner bias as state and, optionally, LayerNorm and a
// residual inside the inner model: f(x) = x + LN(W x + b), LN(u) =
// w * (u - mean(u)) / sqrt(var(u) + eps) + beta over the d features, w and beta
// fixed (diosapp "Test-Time Training (TTT) guide" §3 for f(x) = W x + b; the
// LN-and-residual ablation of PaperTrace "5 · TestingTime 训练与长上下文"
// §3.1).  Without LN, f(x) = W x + b.
//
// Chunked dual form (same page §1.1): every gradient of a chunk is taken at the
// chunk-start (W_c, b_c).  For tokens as columns,
//   U = W_c K + b_c 1^T,  G = dl/dU (column s: through LN, per token),
//   Zpre = M Q + b_m 1^T - G diag(eta) (U o (K^T Q + 1 1^T))   (U: causal mask),
//   Z = Q + LN(Zpre) (or Zpre),  M <- M - G diag(eta) K^T,  b_m <- b_m - G eta,
// in 16-token sub-tiles with M, b_m the running state (= W_c, b_c at a chunk
// start); the "+1" carries the bias through the same causal products.
//
// LN needs all d features of a token, so one workgroup owns a whole (batch,
// head): d/16 waves, wave w holding state rows 16w .. 16w+15 (of W_c and M, all
// columns, in registers).  Every product is a 16 x 16 tile product: on the fp32
// matrix cores with fp32 I/O, on the bf16 ones with bf16 I/O (fp32 operands
// split as hi + lo, about 2^-17 relative per product), in the transposed
// orientation that leaves the state's rows in the lanes (see mfma_f32.h):
//   U^T = K W_c^T,  P^T = Q M^T,  S = K Q^T,  Zpre^T = P^T - S^T (G diag(eta))^T,
//   M^T <- M^T - K^T (G diag(eta))^T,
// so that U, G, P and Zpre all sit as "lane = state row r0 + c, slots = tokens
// 4g .. 4g+3" and the state update lands in the layout the products read.  A
// token's LayerNorm statistics are 16-lane DPP sums inside each wave, combined
// across the waves through LDS ((mean, M2) pairs merged by the parallel-variance
// formula, so each statistic costs one barrier).  The next sub-tile's K, Q, V
// and eta are loaded as raw words while the current one is computed.
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "mfma_f32.h"

namespace ttt {
namespace {

constexpr int kSub = 16;
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a gfx9 buffer resource: raw 32-bit data

// One sub-tile's inputs as loaded: thread t holds 4 consecutive features of one
// token of K, Q and V, and eta of token t % 16.
template <typename TIO>
struct LnTile {
    RawRow<TIO, 4> k, q, v;
    float eta;
};

template <int D>
struct LnLds {
    static constexpr int S = D + 4;   // row stride of the token x feature tiles
    float K[kSub * S];
    float Q[kSub * S];
    float V[kSub * S];
    float eta[kSub];
    // per-wave partial statistics of each token: (mean, M2) of U, (sum g, sum g
    // u-hat) for the LN backward, (mean, M2) of Zpre
    f32x2 stat[3][D / 16][kSub];
};

// one element of the I/O type at byte offset `off` of a range-checked buffer
// (an offset at or past the range's end is dropped by the memory unit)
__device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, int off, float v, float)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), r, off, 0, 0);
}

__device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, int off, float v,
                                              uint16_t)
{
    __builtin_amdgcn_raw_buffer_store_b16((short)f32_to_bf16_bits(v), r, off, 0, 0);
}

// ETA: per-token learning rates (else eta_scalar for every token)
template <typename TIO, int D, bool ETA>
__global__ __launch_bounds__(4 * D) void linear_ln_kernel(
    const TIO* __restrict__ K, const TIO* __restrict__ Q, const TIO* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar, const float* __restrict__ W0,
    const float* __restrict__ b0, const float* __restrict__ lnw, const float* __restrict__ lnb,
    float eps, TIO* __restrict__ Z, float* __restrict__ W_out, float* __restrict__ b_out,
    int H, int T, int chunk)
{
    constexpr int NW = D / 16, NB = D / 16, S = LnLds<D>::S;
    // bf16 I/O: K and Q are exact in bf16 and the tile products run on the bf16
    // matrix cores: those on the state's recurrence (U, the update) split their
    // fp32 operands as hi + lo (mmt), those that only form the bf16 output Z (the
    // read Q M^T, the score-weighted correction) round them to bf16; fp32 I/O
    // keeps fp32 products
    constexpr bool BF = sizeof(TIO) == 2;
    __shared__ __align__(16) LnLds<D> L;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c = lane & 15, g = lane >> 4;
    const int r0 = 16 * wave;   // this wave's state rows
    const int slice = blockIdx.x;
    const int h = slice % H;
    const size_t tok0 = (size_t)slice * T;
    const bool ln = lnw != nullptr;
    const int fs = tid / (D / 4), fj = (tid % (D / 4)) * 4;   // staged token and features

    // state rows r0 + c, columns 16b + 4g .. 16b + 4g + 3 of block b (RL form)
    f32x4 Wc[NB], M[NB];
    {
        const float* w = W0 + ((size_t)slice * D + r0 + c) * D + 4 * g;
#pragma unroll
        for (int b = 0; b < NB; ++b) Wc[b] = M[b] = *reinterpret_cast<const f32x4*>(w + 16 * b);
    }
    float bc = b0[(size_t)slice * D + r0 + c], bm = bc;
    const float lw = ln ? lnw[(size_t)h * D + r0 + c] : 0.f;
    const float lb = ln ? lnb[(size_t)h * D + r0 + c] : 0.f;

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
    auto fetch = [&](LnTile<TIO>& f, int j) {
        int si, t0, len;
        span(j, si, t0, len);
        const size_t off = (tok0 + t0 + min(fs, len - 1)) * D + fj;
        f.k.load(K + off);
        f.q.load(Q + off);
        f.v.load(V + off);
        if constexpr (ETA) f.eta = eta[tok0 + t0 + min(c, len - 1)];
        else f.eta = eta_scalar;
    };
    // Tokens past the sub-tile's end stage the re-read last token as it is: their
    // statistics are their own, every contribution they make is scaled by the
    // masked G diag(eta) (a finite value times zero), and their outputs are never
    // stored.  (A select here would be hoisted onto the freshly loaded registers.)
    auto put = [&](const LnTile<TIO>& f) {
        auto four = [&](const RawRow<TIO, 4>& r) {
            return f32x4{r.at(0), r.at(1), r.at(2), r.at(3)};
        };
        *reinterpret_cast<f32x4*>(L.K + fs * S + fj) = four(f.k);
        *reinterpret_cast<f32x4*>(L.Q + fs * S + fj) = four(f.q);
        *reinterpret_cast<f32x4*>(L.V + fs * S + fj) = four(f.v);
        if (tid < kSub) L.eta[tid] = f.eta;
    };
    // mean and 1/sqrt(var + eps) over the d features of tokens 4g + v, from this
    // wave's 16 rows (lanes c) and the other waves' partials
    auto ln_stats = [&](f32x4 x, int k, f32x4& mean, f32x4& rstd) {
        float sx[4] = {x[0], x[1], x[2], x[3]};
        row_sum16_n(sx);
        float dd[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float dv = x[v] - sx[v] * (1.f / 16.f);
            dd[v] = dv * dv;
        }
        row_sum16_n(dd);
        if (c == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) L.stat[k][wave][4 * g + v] = f32x2{sx[v] * (1.f / 16.f), dd[v]};
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float ms = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) ms += L.stat[k][w][4 * g + v].x;
            const float mu = ms * (1.f / NW);
            float m2 = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const f32x2 p = L.stat[k][w][4 * g + v];
                const float dm = p.x - mu;
                m2 += p.y + 16.f * dm * dm;
            }
            mean[v] = mu;
            rstd[v] = rsqrtf(m2 * (1.f / D) + eps);
        }
    };
    // sums over the d features of tokens 4g + v of two quantities
    auto feature_sums = [&](f32x4 a, f32x4 b, int k, f32x4& sa, f32x4& sb) {
        float r[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        row_sum16_n(r);
        if (c == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) L.stat[k][wave][4 * g + v] = f32x2{r[v], r[4 + v]};
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float x = 0.f, y = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                x += L.stat[k][w][4 * g + v].x;
                y += L.stat[k][w][4 * g + v].y;
            }
            sa[v] = x;
            sb[v] = y;
        }
    };

    // two prefetch slots used alternately at compile-time positions
    LnTile<TIO> bufs[2];
    auto step = [&](int j, auto slot) {
        auto& cur = bufs[decltype(slot)::value];
        auto& nxt = bufs[decltype(slot)::value ^ 1];
        int si, t0, len;
        span(j, si, t0, len);
        __syncthreads();   // the previous sub-tile is done with the tiles and statistics
        put(cur);
        __syncthreads();
        if (j < last) fetch(nxt, j + 1);
        // keep the loads here: sunk below this sub-tile's stores, they would make
        // the next staging wait for those stores too
        __builtin_amdgcn_sched_barrier(0);
        // U^T = K W_c^T (+ b_c), P^T = Q M^T (+ b_m), S = K Q^T, over the features
        f32x4 U = {bc, bc, bc, bc}, P = {bm, bm, bm, bm}, Sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const f32x4 kb = rl<S>(L.K, 16 * b, lane), qb = rl<S>(L.Q, 16 * b, lane);
            U = mmt<BF, true, false>(kb, Wc[b], U);
            P = mmt<BF, true, true>(qb, M[b], P);
            Sc = mmt<BF, true, true>(kb, qb, Sc);
        }
        // causal scores with the bias's +1: writer s = 4g + v, reader t = c
        f32x4 Sm;
#pragma unroll
        for (int v = 0; v < 4; ++v) Sm[v] = (4 * g + v <= c) ? Sc[v] + 1.f : 0.f;
        // G = dl/dU: lane row r0 + c, tokens 4g + v
        const f32x4 kc = cl<S>(L.K, r0, lane), vc = cl<S>(L.V, r0, lane);
        f32x4 G;
        if (ln) {
            f32x4 mu, rs;
            ln_stats(U, 0, mu, rs);
            f32x4 uh, gg, ggu;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                uh[v] = (U[v] - mu[v]) * rs[v];
                gg[v] = lw * (kc[v] + lw * uh[v] + lb - vc[v]);
                ggu[v] = gg[v] * uh[v];
            }
            f32x4 mh, mhu;
            feature_sums(gg, ggu, 1, mh, mhu);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                G[v] = rs[v] * (gg[v] - mh[v] * (1.f / D) - uh[v] * (mhu[v] * (1.f / D)));
        } else {
            G = U - vc;
        }
        // G diag(eta); tokens past the sub-tile's end contribute nothing
        const f32x4 et = *reinterpret_cast<const f32x4*>(L.eta + 4 * g);
        f32x4 Ge;
#pragma unroll
        for (int v = 0; v < 4; ++v) Ge[v] = (4 * g + v < len) ? G[v] * et[v] : 0.f;
        // Zpre^T = P^T - S^T (G eta)^T: A = RL(S^T) = CL(S), B = CL((G eta)^T) = Ge
        const f32x4 Zp = P - mmt<BF, true, true>(Sm, Ge, f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 Zo;
        if (ln) {
            f32x4 mu, rs;
            ln_stats(Zp, 2, mu, rs);
            const f32x4 qc = cl<S>(L.Q, r0, lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) Zo[v] = qc[v] + lw * ((Zp[v] - mu[v]) * rs[v]) + lb;
        } else {
            Zo = Zp;
        }
        // Z[t0 + 4g + v][r0 + c]; tokens past the sub-tile's end fall outside the range
        {
            const auto rz = __builtin_amdgcn_make_buffer_rsrc(
                Z + (tok0 + t0) * D, 0, (int)(len * D * sizeof(TIO)), kBufferFlags);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                buffer_store1(rz, ((4 * g + v) * D + r0 + c) * (int)sizeof(TIO), Zo[v], TIO{});
        }
        // M^T -= K^T (G eta)^T per column block: A = RL(K^T_b) = CL(K_b), B = -Ge
        const f32x4 nGe = -Ge;
#pragma unroll
        for (int b = 0; b < NB; ++b) M[b] = mmt<BF, true, false>(cl<S>(L.K, 16 * b, lane), nGe, M[b]);
        // b_m -= G eta: over the tokens (slots, then lane groups)
        float bs = (Ge[0] + Ge[1]) + (Ge[2] + Ge[3]);
        bs += __shfl_xor(bs, 16);
        bs += __shfl_xor(bs, 32);
        bm -= bs;
        // chunk end: the running state becomes the next chunk-start state
        if (si == nsub - 1 || j == last) {
#pragma unroll
            for (int b = 0; b < NB; ++b) Wc[b] = M[b];
            bc = bm;
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

    {
        float* w = W_out + ((size_t)slice * D + r0 + c) * D + 4 * g;
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(w + 16 * b) = M[b];
    }
    if (g == 0) b_out[(size_t)slice * D + r0 + c] = bm;
}

template <typename TIO>
hipError_t launch_typed(const LinearLnArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)a.BH);
    const TIO* K = static_cast<const TIO*>(a.K);
    const TIO* Q = static_cast<const TIO*>(a.Q);
    const TIO* V = static_cast<const TIO*>(a.V);
    TIO* Z = static_cast<TIO*>(a.Z);
#define TTT_LN_LAUNCH(DD)                                                                    \
    if (a.eta)                                                                               \
        hipLaunchKernelGGL((linear_ln_kernel<TIO, DD, true>), grid, dim3(4 * DD), 0, s, K, Q, \
                           V, a.eta, a.eta_scalar, a.W0, a.b0, a.ln_weight, a.ln_bias, a.eps, \
                           Z, a.W_out, a.b_out, a.H, a.T, a.chunk);                           \
    else                                                                                     \
        hipLaunchKernelGGL((linear_ln_kernel<TIO, DD, false>), grid, dim3(4 * DD), 0, s, K,   \
                           Q, V, a.eta, a.eta_scalar, a.W0, a.b0, a.ln_weight, a.ln_bias,     \
                           a.eps, Z, a.W_out, a.b_out, a.H, a.T, a.chunk)
    switch (a.d) {
    case 16: TTT_LN_LAUNCH(16); break;
    case 32: TTT_LN_LAUNCH(32); break;
    case 64: TTT_LN_LAUNCH(64); break;
    case 128: TTT_LN_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
    }
#undef TTT_LN_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_ln(const LinearLnArgs& a, hipStream_t s)
{
    return a.bf16 ? launch_typed<uint16_t>(a, s) : launch_typed<float>(a, s);
}

}  // namespace ttt
