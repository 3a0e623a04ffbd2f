// TTT-Linear forward scan, generic plan: fp32 vector ALU, any chunk length,
// d <= 128, fp32 or bf16 I/O.
//
// Method: PaperTrace "5 · TestingTime 训练与长上下文" §1.1 and §2.3 — every
// gradient of a chunk is taken at the chunk-start state W_c; token t reads with
// the chunk's updates up to and including its own; the state then moves by
// -sum_s eta_s (W_c k_s - v_s) k_s^T.  In dual form (diosapp "Test-Time Training
// (TTT) guide" §3) a chunk is  E = W_c K - V,  Z = W_c Q - E diag(eta) triu(K^T Q),
// W_{c+1} = W_c - E diag(eta) K^T.
//
// Chunks longer than 16 tokens are walked in 16-token sub-tiles.  E of every
// sub-tile is taken at W_c; the running matrix M = W_c - (updates of earlier
// sub-tiles) gives the cross-sub-tile part of Z exactly, so only a 16 x 16 mask
// is ever formed: Z_tau = M Q_tau - E_tau diag(eta) triu(K_tau^T Q_tau),
// M <- M - E_tau diag(eta) K_tau^T, and W_{c+1} = M at the chunk end.
//
// With the chunk-start read order every token of a chunk reads W_c: Z_tau = W_c Q_tau,
// and the state moves exactly as above -- or, with a momentum state, through
// mom <- beta mom + (1 - beta) (W_c - M), W_{c+1} = W_c - mom at each chunk end.
//
// Work split: one 256-thread workgroup per (batch*head, block of 16 output
// rows).  Output row i of Z and of the state depends only on row i of W0 and
// feature i of V (plus all of K, Q, eta), so row blocks never communicate.
#include "device_common.h"
#include "launch.h"

namespace ttt {
namespace {

constexpr int kTile = 16;        // tokens per sub-tile
constexpr int kRows = 16;        // output rows per workgroup
constexpr int kMaxD = 128;
constexpr int kPad = kMaxD + 1;  // LDS row pitch (odd: no bank conflicts on columns)

template <typename TIO>
__global__ __launch_bounds__(256) void linear_generic_kernel(
    const TIO* __restrict__ K, const TIO* __restrict__ Q, const TIO* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar, const float* W0,
    TIO* __restrict__ Z, float* W_out, int T_all, int d, int chunk, int read_start,
    const int* __restrict__ cu, int H, int total_T, int momentum, float beta,
    const float* __restrict__ mom0, float* __restrict__ mom_out)
{
    __shared__ float sWs[kRows][kPad];   // chunk-start state rows
    __shared__ float sM[kRows][kPad];    // running state rows
    __shared__ float sK[kTile][kPad];
    __shared__ float sQ[kTile][kPad];
    __shared__ float sV[kTile][kRows + 1];
    __shared__ float sE[kRows][kTile + 1];
    __shared__ float sS[kTile][kTile + 1];
    __shared__ float sEta[kTile];
    __shared__ float sMom[kRows][kPad];  // momentum rows (momentum state only)

    const int tid = threadIdx.x;
    const int nrb = (d + kRows - 1) / kRows;
    const int slice = blockIdx.x / nrb;
    const int r0 = (blockIdx.x % nrb) * kRows;
    const int R = min(kRows, d - r0);

    size_t tok0;                                           // first token row of the slice
    int T;
    slice_span(cu, H, total_T, T_all, slice, tok0, T);
    const float* W0s = W0 + (size_t)slice * d * d;
    float* Wos = W_out + (size_t)slice * d * d;

    for (int idx = tid; idx < R * d; idx += 256) {
        int r = idx / d, j = idx % d;
        float w = W0s[(size_t)(r0 + r) * d + j];
        sWs[r][j] = w;
        sM[r][j] = w;
        if (momentum)
            sMom[r][j] = mom0 ? mom0[(size_t)slice * d * d + (size_t)(r0 + r) * d + j] : 0.f;
    }
    __syncthreads();

    // Sub-tiles are walked in order (chunk by chunk); each thread holds its
    // elements of the next sub-tile in registers, loaded while the current one
    // is computed.
    constexpr int kPer = kTile * kMaxD / 256;   // K/Q elements per thread (d <= 128)
    auto next_tile = [&](int c0, int s0, int& nc0, int& ns0) {   // sub-tile after (c0, s0)
        const int c1 = min(T, c0 + chunk);
        if (s0 + kTile < c1) { nc0 = c0; ns0 = s0 + kTile; }
        else { nc0 = c1; ns0 = c1; }
    };
    float rk[kPer], rq[kPer], rv, re;
    auto load_tile = [&](int c0, int s0) {
        const int n = s0 < T ? min(kTile, min(T, c0 + chunk) - s0) : 0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = tid + 256 * e;
            const int i = idx / d, j = idx % d;
            rk[e] = rq[e] = 0.f;
            if (idx < kTile * d && i < n) {
                const size_t off = (tok0 + s0 + i) * d + j;
                rk[e] = io<TIO>::load(K, off);
                rq[e] = io<TIO>::load(Q, off);
            }
        }
        const int i = tid / kRows, r = tid % kRows;
        rv = (i < n && r < R) ? io<TIO>::load(V, (tok0 + s0 + i) * d + r0 + r) : 0.f;
        re = (tid < n) ? (eta ? eta[tok0 + s0 + tid] : eta_scalar) : 0.f;
    };
    int c0 = 0, s0 = 0;
    load_tile(0, 0);
    while (s0 < T) {
        const int c1 = min(T, c0 + chunk);
        const int n = min(kTile, c1 - s0);
        // ---- stage the sub-tile (zeros past its last token) ----
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = tid + 256 * e;
            if (idx < kTile * d) {
                sK[idx / d][idx % d] = rk[e];
                sQ[idx / d][idx % d] = rq[e];
            }
        }
        sV[tid / kRows][tid % kRows] = rv;
        if (tid < kTile) sEta[tid] = re;
        __syncthreads();
        int nc0, ns0;
        next_tile(c0, s0, nc0, ns0);
        load_tile(nc0, ns0);
        {
            // ---- E = W_c K - V  and  S = triu(K^T Q) ----
            {
                int r = tid / kTile, s = tid % kTile;
                if (r < R) {
                    float acc = 0.f;
                    for (int j = 0; j < d; ++j) acc = fmaf(sWs[r][j], sK[s][j], acc);
                    sE[r][s] = acc - sV[s][r];
                }
            }
            {
                int s = tid / kTile, t = tid % kTile;
                float acc = 0.f;
                if (s <= t)
                    for (int j = 0; j < d; ++j) acc = fmaf(sK[s][j], sQ[t][j], acc);
                sS[s][t] = acc;
            }
            __syncthreads();

            // ---- Z = M Q - E diag(eta) S  (chunk-start read: Z = W_c Q) ----
            {
                int t = tid / kRows, r = tid % kRows;
                if (r < R && t < n) {
                    float acc = 0.f, corr = 0.f;
                    if (read_start) {
                        for (int j = 0; j < d; ++j) acc = fmaf(sWs[r][j], sQ[t][j], acc);
                    } else {
                        for (int j = 0; j < d; ++j) acc = fmaf(sM[r][j], sQ[t][j], acc);
                        for (int s = 0; s <= t; ++s)
                            corr = fmaf(sEta[s] * sS[s][t], sE[r][s], corr);
                    }
                    io<TIO>::store(Z, (tok0 + s0 + t) * d + r0 + r, acc - corr);
                }
            }
            __syncthreads();

            // ---- M <- M - E diag(eta) K^T ----
            for (int idx = tid; idx < R * d; idx += 256) {
                int r = idx / d, j = idx % d;
                float acc = 0.f;
                for (int s = 0; s < kTile; ++s) acc = fmaf(sEta[s] * sE[r][s], sK[s][j], acc);
                sM[r][j] -= acc;
            }
            __syncthreads();
        }
        if (s0 + kTile >= c1) {
            // chunk end: the running state becomes the next chunk-start state.  With
            // a momentum state the chunk's gradient g = W_c - M feeds
            // mom <- beta mom + (1 - beta) g, and W_{c+1} = W_c - mom.
            for (int idx = tid; idx < R * d; idx += 256) {
                int r = idx / d, j = idx % d;
                if (momentum) {
                    const float m = beta * sMom[r][j] + (1.f - beta) * (sWs[r][j] - sM[r][j]);
                    sMom[r][j] = m;
                    sM[r][j] = sWs[r][j] - m;
                }
                sWs[r][j] = sM[r][j];
            }
            __syncthreads();
        }
        c0 = nc0;
        s0 = ns0;
    }

    for (int idx = tid; idx < R * d; idx += 256) {
        int r = idx / d, j = idx % d;
        Wos[(size_t)(r0 + r) * d + j] = sM[r][j];
        if (momentum) mom_out[(size_t)slice * d * d + (size_t)(r0 + r) * d + j] = sMom[r][j];
    }
}

}  // namespace

hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t s)
{
    const int nrb = (a.d + kRows - 1) / kRows;
    dim3 grid((unsigned)(a.BH * nrb)), block(256);
    if (a.bf16) {
        hipLaunchKernelGGL(linear_generic_kernel<uint16_t>, grid, block, 0, s,
                           (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V,
                           a.eta, a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.T, a.d,
                           a.chunk, a.read_start, a.cu, a.H, a.total_T, a.momentum, a.beta,
                           a.mom0, a.mom_out);
    } else {
        hipLaunchKernelGGL(linear_generic_kernel<float>, grid, block, 0, s,
                           (const float*)a.K, (const float*)a.Q, (const float*)a.V,
                           a.eta, a.eta_scalar, a.W0, (float*)a.Z, a.W_out, a.T, a.d,
                           a.chunk, a.read_start, a.cu, a.H, a.total_T, a.momentum, a.beta,
                           a.mom0, a.mom_out);
    }
    return hipGetLastError();
}

}  // namespace ttt
