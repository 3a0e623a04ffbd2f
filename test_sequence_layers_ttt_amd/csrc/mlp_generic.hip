// TTT-MLP forward scan, generic plan: fp32 vector ALU, any chunk, d <= 64,
// hidden width 4d.
//
// f(x) = W2 gelu(W1 x + b1) + b2 (diosapp "Test-Time Training (TTT) guide" §3:
// two layers, 4x hidden, GELU), loss 1/2||f(k) - v||^2, chunked update with every
// gradient at the chunk-start parameters and an inclusive read (PaperTrace
// "5 · TestingTime 训练与长上下文" §1.1, §2.3).  Dual form of one 16-token
// sub-tile, columns = tokens, mask U[s,t] = [s <= t]:
//   H = W1 K + b1,  A = gelu(H),  E = W2 A + b2 - V           (forward at P_c)
//   D = (W2^T E) * gelu'(H)                                     (backward)
//   H' = M1 Q + m1 - D diag(eta) (U * (K^T Q + 1)),  A' = gelu(H')
//   Z = M2 A' + m2 - E diag(eta) (U * (A^T A' + 1))
//   M1 -= D diag(eta) K^T, m1 -= D eta, M2 -= E diag(eta) A^T, m2 -= E eta
// where (M1, m1, M2, m2) is the running state: the chunk-start parameters minus
// the updates of the chunk's earlier sub-tiles.  The "+1" terms come from the
// biases and are dropped for a model without that bias.
//
// One 256-thread workgroup per (batch, head): the MLP state does not split by
// output rows.  The running state lives in the output buffers; chunks longer
// than one sub-tile keep a chunk-start copy in the workspace.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace ttt {
namespace {

constexpr int kTile = 16;

__device__ __forceinline__ float gelu_f(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_prime_f(float x)
{
    return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) +
           x * 0.39894228040143268f * expf(-0.5f * x * x);
}

struct Smem {
    float* K;    // [16][d+1]
    float* Q;    // [16][d+1]
    float* V;    // [16][d+1]
    float* eta;  // [16]
    float* A;    // [hd][17]  gelu(H)
    float* G;    // [hd][17]  gelu'(H)
    float* D;    // [hd][17]  delta
    float* Aq;   // [hd][17]  H' then gelu(H')
    float* E;    // [d][17]
    float* S1;   // [16][17]
    float* S2;   // [16][17]
};

__host__ __device__ inline size_t smem_floats(int d)
{
    int hd = 4 * d;
    return (size_t)3 * kTile * (d + 1) + kTile + (size_t)4 * hd * 17 + (size_t)d * 17 + 2 * 16 * 17;
}

template <typename TIO>
__global__ __launch_bounds__(256) void mlp_generic_kernel(
    const TIO* __restrict__ K, const TIO* __restrict__ Q, const TIO* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar,
    const float* W1_0, const float* b1_0, const float* W2_0, const float* b2_0,
    TIO* __restrict__ Z, float* W1r, float* b1r, float* W2r, float* b2r,
    float* ws, int T, int d, int chunk)
{
    extern __shared__ float smem[];
    const int hd = 4 * d;
    const int dp = d + 1;
    Smem s;
    s.K = smem;
    s.Q = s.K + kTile * dp;
    s.V = s.Q + kTile * dp;
    s.eta = s.V + kTile * dp;
    s.A = s.eta + kTile;
    s.G = s.A + hd * 17;
    s.D = s.G + hd * 17;
    s.Aq = s.D + hd * 17;
    s.E = s.Aq + hd * 17;
    s.S1 = s.E + d * 17;
    s.S2 = s.S1 + 16 * 17;

    const int tid = threadIdx.x;
    const int slice = blockIdx.x;
    const size_t n1 = (size_t)hd * d;
    const size_t tok0 = (size_t)slice * T;
    const bool has_b1 = b1_0 != nullptr, has_b2 = b2_0 != nullptr;

    // running state (output buffers), initialised from the inputs
    float* W1 = W1r + slice * n1;
    float* W2 = W2r + slice * n1;
    float* b1 = has_b1 ? b1r + (size_t)slice * hd : nullptr;
    float* b2 = has_b2 ? b2r + (size_t)slice * d : nullptr;
    for (size_t i = tid; i < n1; i += 256) {
        W1[i] = W1_0[slice * n1 + i];
        W2[i] = W2_0[slice * n1 + i];
    }
    if (has_b1) for (int i = tid; i < hd; i += 256) b1[i] = b1_0[(size_t)slice * hd + i];
    if (has_b2) for (int i = tid; i < d; i += 256) b2[i] = b2_0[(size_t)slice * d + i];

    // chunk-start parameters: the running state itself when a chunk is one
    // sub-tile, else a copy in the workspace
    const bool copy = chunk > kTile;
    const size_t per = 2 * n1 + hd + d;
    float* W1s = copy ? ws + slice * per : W1;
    float* W2s = copy ? W1s + n1 : W2;
    float* b1s = copy ? W2s + n1 : b1;
    float* b2s = copy ? b1s + hd : b2;
    __syncthreads();

    for (int c0 = 0; c0 < T; c0 += chunk) {
        const int c1 = min(T, c0 + chunk);
        if (copy) {
            for (size_t i = tid; i < n1; i += 256) {
                W1s[i] = W1[i];
                W2s[i] = W2[i];
            }
            for (int i = tid; i < hd; i += 256) b1s[i] = has_b1 ? b1[i] : 0.f;
            for (int i = tid; i < d; i += 256) b2s[i] = has_b2 ? b2[i] : 0.f;
            __syncthreads();
        }
        for (int s0 = c0; s0 < c1; s0 += kTile) {
            const int n = min(kTile, c1 - s0);
            for (int idx = tid; idx < kTile * d; idx += 256) {
                int i = idx / d, j = idx % d;
                float kv = 0.f, qv = 0.f, vv = 0.f;
                if (i < n) {
                    size_t off = (tok0 + s0 + i) * d + j;
                    kv = io<TIO>::load(K, off);
                    qv = io<TIO>::load(Q, off);
                    vv = io<TIO>::load(V, off);
                }
                s.K[i * dp + j] = kv;
                s.Q[i * dp + j] = qv;
                s.V[i * dp + j] = vv;
            }
            if (tid < kTile) s.eta[tid] = (tid < n) ? (eta ? eta[tok0 + s0 + tid] : eta_scalar) : 0.f;
            __syncthreads();

            // H = W1s K + b1s ; A = gelu(H) ; G = gelu'(H)
            for (int idx = tid; idx < hd * kTile; idx += 256) {
                int u = idx / kTile, t = idx % kTile;
                float acc = has_b1 ? b1s[u] : 0.f;
                for (int j = 0; j < d; ++j) acc = fmaf(W1s[(size_t)u * d + j], s.K[t * dp + j], acc);
                s.A[u * 17 + t] = gelu_f(acc);
                s.G[u * 17 + t] = gelu_prime_f(acc);
            }
            __syncthreads();
            // E = W2s A + b2s - V   (zero for padding tokens)
            for (int idx = tid; idx < d * kTile; idx += 256) {
                int i = idx / kTile, t = idx % kTile;
                float acc = has_b2 ? b2s[i] : 0.f;
                for (int u = 0; u < hd; ++u) acc = fmaf(W2s[(size_t)i * hd + u], s.A[u * 17 + t], acc);
                s.E[i * 17 + t] = (t < n) ? acc - s.V[t * dp + i] : 0.f;
            }
            // S1 = U * (K^T Q + 1)
            {
                int a = tid / kTile, t = tid % kTile;
                float acc = 0.f;
                if (a <= t) {
                    for (int j = 0; j < d; ++j) acc = fmaf(s.K[a * dp + j], s.Q[t * dp + j], acc);
                    if (has_b1) acc += 1.f;
                }
                s.S1[a * 17 + t] = acc;
            }
            __syncthreads();
            // D = (W2s^T E) * G
            for (int idx = tid; idx < hd * kTile; idx += 256) {
                int u = idx / kTile, t = idx % kTile;
                float acc = 0.f;
                for (int i = 0; i < d; ++i) acc = fmaf(W2s[(size_t)i * hd + u], s.E[i * 17 + t], acc);
                s.D[u * 17 + t] = acc * s.G[u * 17 + t];
            }
            __syncthreads();
            // H' = M1 Q + m1 - D diag(eta) S1 ;  A' = gelu(H')
            for (int idx = tid; idx < hd * kTile; idx += 256) {
                int u = idx / kTile, t = idx % kTile;
                float acc = has_b1 ? b1[u] : 0.f;
                for (int j = 0; j < d; ++j) acc = fmaf(W1[(size_t)u * d + j], s.Q[t * dp + j], acc);
                float corr = 0.f;
                for (int a = 0; a <= t; ++a) corr = fmaf(s.eta[a] * s.S1[a * 17 + t], s.D[u * 17 + a], corr);
                s.Aq[u * 17 + t] = gelu_f(acc - corr);
            }
            __syncthreads();
            // S2 = U * (A^T A' + 1)
            {
                int a = tid / kTile, t = tid % kTile;
                float acc = 0.f;
                if (a <= t) {
                    for (int u = 0; u < hd; ++u) acc = fmaf(s.A[u * 17 + a], s.Aq[u * 17 + t], acc);
                    if (has_b2) acc += 1.f;
                }
                s.S2[a * 17 + t] = acc;
            }
            __syncthreads();
            // Z = M2 A' + m2 - E diag(eta) S2
            for (int idx = tid; idx < d * kTile; idx += 256) {
                int t = idx / d, i = idx % d;
                if (t < n) {
                    float acc = has_b2 ? b2[i] : 0.f;
                    for (int u = 0; u < hd; ++u) acc = fmaf(W2[(size_t)i * hd + u], s.Aq[u * 17 + t], acc);
                    float corr = 0.f;
                    for (int a = 0; a <= t; ++a) corr = fmaf(s.eta[a] * s.S2[a * 17 + t], s.E[i * 17 + a], corr);
                    io<TIO>::store(Z, (tok0 + s0 + t) * d + i, acc - corr);
                }
            }
            __syncthreads();
            // running-state update
            for (size_t idx = tid; idx < n1; idx += 256) {
                int u = (int)(idx / d), j = (int)(idx % d);
                float acc = 0.f;
                for (int t = 0; t < kTile; ++t) acc = fmaf(s.eta[t] * s.D[u * 17 + t], s.K[t * dp + j], acc);
                W1[idx] -= acc;
            }
            for (size_t idx = tid; idx < n1; idx += 256) {
                int i = (int)(idx / hd), u = (int)(idx % hd);
                float acc = 0.f;
                for (int t = 0; t < kTile; ++t) acc = fmaf(s.eta[t] * s.E[i * 17 + t], s.A[u * 17 + t], acc);
                W2[idx] -= acc;
            }
            if (has_b1)
                for (int u = tid; u < hd; u += 256) {
                    float acc = 0.f;
                    for (int t = 0; t < kTile; ++t) acc = fmaf(s.eta[t], s.D[u * 17 + t], acc);
                    b1[u] -= acc;
                }
            if (has_b2)
                for (int i = tid; i < d; i += 256) {
                    float acc = 0.f;
                    for (int t = 0; t < kTile; ++t) acc = fmaf(s.eta[t], s.E[i * 17 + t], acc);
                    b2[i] -= acc;
                }
            __syncthreads();
        }
    }
}

}  // namespace

size_t mlp_generic_workspace(int BH, int T, int d, int chunk)
{
    (void)T;
    if (chunk <= kTile) return 0;
    size_t hd = 4 * (size_t)d;
    return (size_t)BH * (2 * hd * d + hd + d) * sizeof(float);
}

hipError_t launch_mlp_generic(const MlpArgs& a, hipStream_t s)
{
    const size_t lds = smem_floats(a.d) * sizeof(float);
    dim3 grid((unsigned)a.BH), block(256);
    if (a.bf16) {
        auto k = mlp_generic_kernel<uint16_t>;
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k, grid, block, lds, s, (const uint16_t*)a.K, (const uint16_t*)a.Q,
                           (const uint16_t*)a.V, a.eta, a.eta_scalar, a.W1, a.b1, a.W2, a.b2,
                           (uint16_t*)a.Z, a.W1_out, a.b1_out, a.W2_out, a.b2_out,
                           (float*)a.workspace, a.T, a.d, a.chunk);
    } else {
        auto k = mlp_generic_kernel<float>;
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k, grid, block, lds, s, (const float*)a.K, (const float*)a.Q,
                           (const float*)a.V, a.eta, a.eta_scalar, a.W1, a.b1, a.W2, a.b2,
                           (float*)a.Z, a.W1_out, a.b1_out, a.W2_out, a.b2_out,
                           (float*)a.workspace, a.T, a.d, a.chunk);
    }
    return hipGetLastError();
}

}  // namespace ttt
