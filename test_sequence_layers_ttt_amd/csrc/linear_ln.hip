// TTT-Linear with the inner bias as state and, optionally, LayerNorm and a
// residual inside the inner model: f(x) = x + LN(W x + b), LN(u) =
// w * (u - mean(u)) / sqrt(var(u) + eps) + beta over the d features, w and beta
// fixed (diosapp "Test-Time Training (TTT) guide" §3 for f(x) = W x + b; the
// LN-and-residual ablation discussed in PaperTrace "5 · TestingTime
// 训练与长上下文").  Without LN, f(x) = W x + b.
//
// Chunked dual form (same page §1.1): every gradient of a chunk is taken at the
// chunk-start (W_c, b_c).  For tokens as columns,
//   U = W_c K + b_c 1^T,  G = dl/dU (column s: through LN, per token),
//   Zpre = M Q + b_m 1^T - G diag(eta) (U o (K^T Q + 1 1^T))   (U: causal mask),
//   Z = Q + LN(Zpre) (or Zpre),  M <- M - G diag(eta) K^T,  b_m <- b_m - G eta,
// in 16-token sub-tiles with M, b_m the running state (= W_c, b_c at a chunk
// start); the "+1" carries the bias through the same causal products.
//
// LN needs all d features of a token, so one workgroup (256 threads, 512 at
// d = 128) owns a whole (batch, head) state, fp32 on the vector ALUs.  Thread
// (row i, part p) holds columns [p*C, (p+1)*C) of row i of W_c and M
// (C = d*d/threads); row sums are butterfly reductions over the threads of a
// row, and per-token statistics reductions over threads/16 lanes.
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace ttt {
namespace {

constexpr int kSub = 16;

// sum over the N consecutive lanes of a group (N a power of two <= 32); every
// lane of the group receives the sum
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int o = N / 2; o >= 1; o /= 2) x += __shfl_xor(x, o, N);
    return x;
}

template <int D>
constexpr int ln_threads()
{
    return D == 128 ? 512 : 256;
}

// ETA: per-token learning rates (else eta_scalar for every token)
template <typename TIO, int D, bool ETA>
__global__ __launch_bounds__(ln_threads<D>()) void linear_ln_kernel(
    const TIO* __restrict__ K, const TIO* __restrict__ Q, const TIO* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar, const float* __restrict__ W0,
    const float* __restrict__ b0, const float* __restrict__ lnw, const float* __restrict__ lnb,
    float eps, TIO* __restrict__ Z, float* __restrict__ W_out, float* __restrict__ b_out,
    int H, int T, int chunk)
{
    constexpr int NT = ln_threads<D>();
    constexpr int TPR = NT / D;           // threads per state row
    constexpr int C = D / TPR;            // columns per thread
    constexpr int SP = D + 4;             // LDS row pitch: 16-byte rows, columns on distinct banks
    constexpr int PRE = kSub * D / NT;    // elements of each staged tile per thread
    constexpr int LPT = NT / kSub;        // lanes per token in the per-token layout
    constexpr int FPL = D / LPT;          // features per lane there
    __shared__ __align__(16) float sK[kSub][SP];
    __shared__ __align__(16) float sQ[kSub][SP];
    __shared__ __align__(16) float sV[kSub][SP];
    __shared__ float sU[kSub][SP];        // U, then G             [token][feature]
    __shared__ float sP[kSub][SP];        // M Q + b_m, then Zpre  [token][feature]
    __shared__ float sS[kSub][kSub + 1];  // k_s . q_t + 1 for s <= t, else 0
    __shared__ float sEta[kSub];
    __shared__ float sbc[D], sbm[D], sw[D], sbeta[D];

    const int tid = threadIdx.x;
    const int slice = blockIdx.x;
    const int row = tid / TPR, part = tid % TPR, col0 = part * C;
    const int tt = tid / LPT, l16 = tid % LPT;   // per-token layout: token tt, lane l16
    const bool ln = lnw != nullptr;
    const size_t tok0 = (size_t)slice * T;
    const int h = slice % H;

    float wc[C], wm[C];
    {
        const float* w = W0 + ((size_t)slice * D + row) * D + col0;
#pragma unroll
        for (int j = 0; j < C; ++j) wc[j] = wm[j] = w[j];
    }
    for (int i = tid; i < D; i += NT) {
        sbc[i] = sbm[i] = b0[(size_t)slice * D + i];
        sw[i] = ln ? lnw[(size_t)h * D + i] : 0.f;
        sbeta[i] = ln ? lnb[(size_t)h * D + i] : 0.f;
    }

    // The next sub-tile's K, Q, V and eta are loaded into registers, as the
    // loaded words, while the current one is computed.  Thread tid takes PRE
    // consecutive features of token fs; tokens past the sub-tile's end re-read
    // its last token and are staged as zeros, so every path issues the same
    // loads and only the staging waits for them.
    const int fs = tid * PRE / D, fj = tid * PRE % D;
    RawRow<TIO, PRE> rk, rq, rv;
    float re = eta_scalar;
    auto fetch = [&](int s0, int n) {
        const size_t off = (tok0 + s0 + min(fs, n - 1)) * D + fj;
        rk.load(K + off);
        rq.load(Q + off);
        rv.load(V + off);
        if constexpr (ETA) re = eta[tok0 + s0 + min(tid % kSub, n - 1)];
    };
    // sub-tile after the one at s0 (chunk starting at c0)
    auto next = [&](int c0, int s0, int& nc0, int& ns0) {
        const int c1 = min(T, c0 + chunk);
        if (s0 + kSub < c1) { nc0 = c0; ns0 = s0 + kSub; }
        else { nc0 = c1; ns0 = c1; }
    };
    fetch(0, min(kSub, min(T, chunk)));

    for (int c0 = 0; c0 < T; c0 += chunk) {
        const int c1 = min(T, c0 + chunk);
        for (int s0 = c0; s0 < c1; s0 += kSub) {
            const int n = min(kSub, c1 - s0);
            __syncthreads();   // previous sub-tile done with the LDS tiles
            // ---- stage the prefetched K, Q, V and eta, then fetch the next ----
            {
                const bool ok = fs < n;
#pragma unroll
                for (int i = 0; i < PRE; ++i) {
                    sK[fs][fj + i] = ok ? rk.at(i) : 0.f;
                    sQ[fs][fj + i] = ok ? rq.at(i) : 0.f;
                    sV[fs][fj + i] = ok ? rv.at(i) : 0.f;
                }
            }
            if (tid < kSub) sEta[tid] = tid < n ? re : 0.f;
            {
                int nc0, ns0;
                next(c0, s0, nc0, ns0);
                if (ns0 < T) fetch(ns0, min(kSub, min(T, nc0 + chunk) - ns0));
            }
            __syncthreads();
            // ---- U = W_c K + b_c and P = M Q + b_m (row sums over the row's threads) ----
#pragma unroll 2
            for (int s = 0; s < kSub; ++s) {
                float u = 0.f, p = 0.f;
                if constexpr (C % 4 == 0) {
#pragma unroll
                    for (int j = 0; j < C; j += 4) {
                        const float4 k4 = *reinterpret_cast<const float4*>(&sK[s][col0 + j]);
                        const float4 q4 = *reinterpret_cast<const float4*>(&sQ[s][col0 + j]);
                        u = fmaf(wc[j], k4.x, u); u = fmaf(wc[j + 1], k4.y, u);
                        u = fmaf(wc[j + 2], k4.z, u); u = fmaf(wc[j + 3], k4.w, u);
                        p = fmaf(wm[j], q4.x, p); p = fmaf(wm[j + 1], q4.y, p);
                        p = fmaf(wm[j + 2], q4.z, p); p = fmaf(wm[j + 3], q4.w, p);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < C; ++j) {
                        u = fmaf(wc[j], sK[s][col0 + j], u);
                        p = fmaf(wm[j], sQ[s][col0 + j], p);
                    }
                }
                u = group_sum<TPR>(u);
                p = group_sum<TPR>(p);
                if (part == 0) {
                    sU[s][row] = u + sbc[row];
                    sP[s][row] = p + sbm[row];
                }
            }
            // ---- causal scores (with the bias's +1) ----
            if (tid < kSub * kSub) {
                const int s = tid >> 4, t = tid & 15;
                float acc = 0.f;
                if (s <= t && t < n) {
                    for (int j = 0; j < D; ++j) acc = fmaf(sK[s][j], sQ[t][j], acc);
                    acc += 1.f;
                }
                sS[s][t] = acc;
            }
            __syncthreads();
            // ---- G = dl/dU per token (token tt, features l16 + 16 m) ----
            {
                float u[FPL], g[FPL];
                float mu = 0.f, var = 0.f;
#pragma unroll
                for (int m = 0; m < FPL; ++m) u[m] = sU[tt][l16 + LPT * m];
                if (ln) {
#pragma unroll
                    for (int m = 0; m < FPL; ++m) mu += u[m];
                    mu = group_sum<LPT>(mu) / D;
#pragma unroll
                    for (int m = 0; m < FPL; ++m) var += (u[m] - mu) * (u[m] - mu);
                    var = group_sum<LPT>(var) / D;
                    const float rs = rsqrtf(var + eps);
                    float mh = 0.f, mhu = 0.f;
#pragma unroll
                    for (int m = 0; m < FPL; ++m) {
                        const int i = l16 + LPT * m;
                        const float uh = (u[m] - mu) * rs;
                        const float r = sK[tt][i] + sw[i] * uh + sbeta[i] - sV[tt][i];
                        g[m] = sw[i] * r;
                        mh += g[m];
                        mhu += g[m] * uh;
                        u[m] = uh;
                    }
                    mh = group_sum<LPT>(mh) / D;
                    mhu = group_sum<LPT>(mhu) / D;
#pragma unroll
                    for (int m = 0; m < FPL; ++m) g[m] = rs * (g[m] - mh - u[m] * mhu);
                } else {
#pragma unroll
                    for (int m = 0; m < FPL; ++m) g[m] = u[m] - sV[tt][l16 + LPT * m];
                }
                __syncthreads();   // every lane has read U
#pragma unroll
                for (int m = 0; m < FPL; ++m) sU[tt][l16 + LPT * m] = tt < n ? g[m] : 0.f;
            }
            __syncthreads();
            // ---- Zpre = P - G diag(eta) S, then Z = Q + LN(Zpre) (token tt) ----
            {
                float zp[FPL];
                float mu = 0.f, var = 0.f;
#pragma unroll
                for (int m = 0; m < FPL; ++m) {
                    const int i = l16 + LPT * m;
                    float acc = sP[tt][i];
                    for (int s = 0; s <= tt; ++s) acc = fmaf(-sEta[s] * sS[s][tt], sU[s][i], acc);
                    zp[m] = acc;
                    mu += acc;
                }
                if (ln) {
                    mu = group_sum<LPT>(mu) / D;
#pragma unroll
                    for (int m = 0; m < FPL; ++m) var += (zp[m] - mu) * (zp[m] - mu);
                    var = group_sum<LPT>(var) / D;
                    const float rs = rsqrtf(var + eps);
#pragma unroll
                    for (int m = 0; m < FPL; ++m) {
                        const int i = l16 + LPT * m;
                        zp[m] = sQ[tt][i] + sw[i] * ((zp[m] - mu) * rs) + sbeta[i];
                    }
                }
                if (tt < n) {
#pragma unroll
                    for (int m = 0; m < FPL; ++m)
                        io<TIO>::store(Z, (tok0 + s0 + tt) * D + l16 + LPT * m, zp[m]);
                }
            }
            // ---- M -= G diag(eta) K^T, b_m -= G eta ----
#pragma unroll 2
            for (int s = 0; s < kSub; ++s) {
                const float f = sEta[s] * sU[s][row];
                if constexpr (C % 4 == 0) {
#pragma unroll
                    for (int j = 0; j < C; j += 4) {
                        const float4 k4 = *reinterpret_cast<const float4*>(&sK[s][col0 + j]);
                        wm[j] = fmaf(-f, k4.x, wm[j]);
                        wm[j + 1] = fmaf(-f, k4.y, wm[j + 1]);
                        wm[j + 2] = fmaf(-f, k4.z, wm[j + 2]);
                        wm[j + 3] = fmaf(-f, k4.w, wm[j + 3]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < C; ++j) wm[j] = fmaf(-f, sK[s][col0 + j], wm[j]);
                }
            }
            __syncthreads();   // every lane has read b_m through sP's producers
            if (part == 0) {
                float acc = 0.f;
                for (int s = 0; s < kSub; ++s) acc = fmaf(sEta[s], sU[s][row], acc);
                sbm[row] -= acc;
            }
        }
        // chunk end: the running state becomes the next chunk-start state
#pragma unroll
        for (int j = 0; j < C; ++j) wc[j] = wm[j];
        __syncthreads();
        for (int i = tid; i < D; i += NT) sbc[i] = sbm[i];
    }
    __syncthreads();
    {
        float* w = W_out + ((size_t)slice * D + row) * D + col0;
#pragma unroll
        for (int j = 0; j < C; ++j) w[j] = wm[j];
    }
    for (int i = tid; i < D; i += NT) b_out[(size_t)slice * D + i] = sbm[i];
}

template <typename TIO>
hipError_t launch_typed(const LinearLnArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)a.BH);
    const TIO* K = static_cast<const TIO*>(a.K);
    const TIO* Q = static_cast<const TIO*>(a.Q);
    const TIO* V = static_cast<const TIO*>(a.V);
    TIO* Z = static_cast<TIO*>(a.Z);
#define TTT_LN_LAUNCH(DD)                                                                      \
    if (a.eta)                                                                                 \
        hipLaunchKernelGGL((linear_ln_kernel<TIO, DD, true>), grid, dim3(ln_threads<DD>()), 0, \
                           s, K, Q, V, a.eta, a.eta_scalar, a.W0, a.b0, a.ln_weight,            \
                           a.ln_bias, a.eps, Z, a.W_out, a.b_out, a.H, a.T, a.chunk);           \
    else                                                                                       \
        hipLaunchKernelGGL((linear_ln_kernel<TIO, DD, false>), grid, dim3(ln_threads<DD>()),   \
                           0, s, K, Q, V, a.eta, a.eta_scalar, a.W0, a.b0, a.ln_weight,         \
                           a.ln_bias, a.eps, Z, a.W_out, a.b_out, a.H, a.T, a.chunk)
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
