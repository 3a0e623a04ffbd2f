// Internal launchers, one per kernel plan.  The C ABI (api.cpp) validates every
// argument before calling these; they only size the grid and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ttt {

struct LinearArgs {
    const void* K;
    const void* Q;
    const void* V;
    const float* eta;      // [BH, T] or nullptr
    float eta_scalar;
    const float* W0;       // [BH, d, d]
    void* Z;
    float* W_out;
    int BH, T, d, chunk;
    int bf16;              // 1: K/Q/V/Z are bf16, 0: fp32
    int read_start;        // 1: every token reads with its chunk-start state
    void* workspace;
    size_t workspace_bytes;
    // momentum state (chunk-start reads): M <- beta M + (1 - beta) grad_c,
    // W <- W - M per chunk; mom0 may be null (zero)
    int momentum;
    float beta;
    const float* mom0;     // [BH, d, d] or nullptr
    float* mom_out;        // [BH, d, d]
    // packed documents: when cu is set, slice s = (document s / H, head s % H) reads
    // tokens [cu[doc], cu[doc + 1]) of head h's rows of [H, total_T, d] (clamped to
    // [0, total_T]); T is then unused
    const int* cu;
    int H, total_T;
};

// Token range of one slice: its first row in the packed arrays and its length.
__device__ __forceinline__ void slice_span(const int* cu, int H, int total_T, int T, int slice,
                                           size_t& tok0, int& len)
{
    if (!cu) {
        tok0 = (size_t)slice * T;
        len = T;
        return;
    }
    const int doc = slice / H, h = slice - doc * H;
    const int st = min(max(cu[doc], 0), total_T);
    const int en = min(max(cu[doc + 1], st), total_T);
    tok0 = (size_t)h * total_T + st;
    len = en - st;
}

struct MlpArgs {
    const void* K;
    const void* Q;
    const void* V;
    const float* eta;
    float eta_scalar;
    const float* W1;       // [BH, 4d, d]
    const float* b1;       // [BH, 4d] or nullptr
    const float* W2;       // [BH, d, 4d]
    const float* b2;       // [BH, d] or nullptr
    void* Z;
    float* W1_out;
    float* b1_out;
    float* W2_out;
    float* b2_out;
    int BH, T, d, chunk;
    int bf16;
    void* workspace;
    size_t workspace_bytes;
};

// fp32 vector-ALU dual form, any chunk, d <= 128, either read order.
hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t s);

// bf16 MFMA path for chunk <= 16 or a multiple of 16; d in {32, 64, 128}.  Packed
// documents: chunk <= 16 only.
bool linear_mfma_supported(int d, int chunk, int bf16);
hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s);

// Segments along T for chunk-16 heads at d = 64 that leave compute units idle:
// each slice's sequence in S segments (S * slices workgroups of four waves);
// segment 0 scans while the others form their affine maps, a combine gives every
// segment its start state, and segments 1 .. S-1 scan again from it.  The
// workspace holds W_B, A and W_start [BH, S, d, d] fp32.
bool linear_seg_supported(int BH, int T, int d, int chunk, int bf16);
bool linear_seg_preferred(int BH, int T);
size_t linear_seg_workspace(int BH, int T, int d);
hipError_t launch_linear_seg(const LinearArgs& a, hipStream_t s);

// fp32 I/O on the fp32 matrix cores: one wave per (batch*head, 16-row block), any
// chunk, d in {16, 32, 64, 128}, the inclusive read; part of the MFMA plan.
bool linear_f32_supported(int d);
hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t s);

// Chunks of exactly 16 tokens, one workgroup of d/16 waves per (batch, head)
// sharing each chunk's K/Q tile through LDS; part of the MFMA plan.
bool linear_coop_supported(int d, int chunk, int bf16);
hipError_t launch_linear_coop(const LinearArgs& a, hipStream_t s);

// three-stage large-chunk path; chunk a multiple of 32, >= 128; d in {64, 128}; bf16;
// either read order.
bool linear_bigchunk_supported(int d, int chunk, int bf16);
size_t linear_bigchunk_workspace(int BH, int T, int d, int chunk);
hipError_t launch_linear_bigchunk(const LinearArgs& a, hipStream_t s);

struct LinearLnArgs {
    const void* K;
    const void* Q;
    const void* V;
    const float* eta;
    float eta_scalar;
    const float* W0;         // [BH, d, d]
    const float* b0;         // [BH, d]
    const float* ln_weight;  // [H, d] or nullptr (no LayerNorm, no residual)
    const float* ln_bias;    // [H, d] or nullptr
    float eps;
    void* Z;
    float* W_out;
    float* b_out;
    int BH, H, T, d, chunk;
    int bf16;
};

// TTT-Linear with the inner bias and optional LayerNorm + residual inside f:
// fp32 matrix cores, one workgroup of d/16 waves per (batch, head), any chunk,
// d <= 128.
hipError_t launch_linear_ln(const LinearLnArgs& a, hipStream_t s);

struct LinearBwdArgs {
    const void* K;
    const void* Q;
    const void* V;
    const float* eta;      // [BH, T] or nullptr
    float eta_scalar;
    const float* W0;       // [BH, d, d]
    const void* dZ;        // [BH, T, d] in the I/O type
    const float* dW_T;     // [BH, d, d] or nullptr (zero)
    void* dK;              // outputs [BH, T, d] in the I/O type
    void* dQ;
    void* dV;
    float* deta;           // [BH, T] or nullptr (not written)
    float* dW0;            // [BH, d, d]
    int BH, T, d, chunk;
    int bf16;
    void* workspace;
    size_t workspace_bytes;
};

// Backward pass of TTT-Linear (fp32 matrix cores), d in {16, 32, 64, 128}, any
// chunk; the workspace holds the chunk-start states and, with bf16 I/O, the fp32
// sums of dK and dQ.
size_t linear_bwd_align(size_t bytes);
size_t linear_bwd_workspace(int BH, int T, int d, int chunk, bool bf16);
hipError_t launch_linear_bwd(const LinearBwdArgs& a, hipStream_t s);

// Streaming continuation from a carried (chunk-start state, in-chunk update) pair;
// fp32 vector ALU, d <= 128.  a.W_out is the chunk-start state, updated in place,
// and a.T the number of new tokens.
hipError_t launch_linear_step(const LinearArgs& a, float* G, int pos, hipStream_t s);

// TTT-MLP: generic fp32 path (d <= 64) and the bf16 MFMA path (d == 64, chunk <= 16).
size_t mlp_generic_workspace(int BH, int T, int d, int chunk);
hipError_t launch_mlp_generic(const MlpArgs& a, hipStream_t s);
bool mlp_mfma_supported(int d, int chunk, int bf16);
hipError_t launch_mlp_mfma(const MlpArgs& a, hipStream_t s);

}  // namespace ttt
