// C ABI of libttt_amd.so (declared in include/ttt.h).
//
// Every argument is validated here, on the host, before any HIP call; a failed
// check returns a negative status and enqueues nothing.  Plan selection picks a
// kernel for the shape; the launchers in the kernel files only size grids.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "ttt.h"
#include "launch.h"

using namespace ttt;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dims_ok(int B, int H, int T, int d, int chunk)
{
    if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || chunk <= 0) return false;
    // keep every element index inside 2^62 and the grid inside 2^31 workgroups
    long double n = (long double)B * H * T * d;
    return n < 4.0e18L && (long double)B * H * 64 < 2.0e9L;
}

int linear_plan(int B, int H, int T, int d, int chunk, int io_dtype, int plan,
                int read_mode = TTT_READ_INCLUSIVE)
{
    if (!dims_ok(B, H, T, d, chunk)) return TTT_ERR_INVALID_ARG;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARG;
    if (plan < TTT_PLAN_AUTO || plan > TTT_PLAN_SPLIT) return TTT_ERR_INVALID_ARG;
    if (read_mode != TTT_READ_INCLUSIVE && read_mode != TTT_READ_CHUNK_START)
        return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    const int bf16 = io_dtype == TTT_DTYPE_BF16;
    // the small-chunk matrix-core kernels implement the inclusive read only: bf16
    // I/O on the bf16 matrix cores, fp32 I/O on the fp32 ones (any chunk)
    const bool mfma = read_mode == TTT_READ_INCLUSIVE &&
                      (bf16 ? linear_mfma_supported(d, chunk, bf16) : linear_f32_supported(d));
    const bool big = linear_bigchunk_supported(d, chunk, bf16);
    const bool split = read_mode == TTT_READ_INCLUSIVE &&
                       linear_seg_supported(B * H, T, d, chunk, bf16);
    switch (plan) {
    case TTT_PLAN_GENERIC: return TTT_PLAN_GENERIC;
    case TTT_PLAN_MFMA: return mfma ? TTT_PLAN_MFMA : TTT_ERR_UNSUPPORTED;
    case TTT_PLAN_BIGCHUNK: return big ? TTT_PLAN_BIGCHUNK : TTT_ERR_UNSUPPORTED;
    case TTT_PLAN_SPLIT: return split ? TTT_PLAN_SPLIT : TTT_ERR_UNSUPPORTED;
    default: break;
    }
    // chunks of 128+ tokens: the three-stage path spreads the chunks over the GPU
    if (big) return TTT_PLAN_BIGCHUNK;
    // few heads: segments along T use the compute units the heads leave idle
    if (split && linear_seg_preferred(B * H, T)) return TTT_PLAN_SPLIT;
    if (mfma) return TTT_PLAN_MFMA;
    return TTT_PLAN_GENERIC;
}

int mlp_plan(int B, int H, int T, int d, int chunk, int io_dtype, int plan)
{
    if (!dims_ok(B, H, T, d, chunk)) return TTT_ERR_INVALID_ARG;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARG;
    if (plan < TTT_PLAN_AUTO || plan > TTT_PLAN_SPLIT) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64) return TTT_ERR_UNSUPPORTED;
    const bool mfma = mlp_mfma_supported(d, chunk, io_dtype == TTT_DTYPE_BF16);
    switch (plan) {
    case TTT_PLAN_GENERIC: return TTT_PLAN_GENERIC;
    case TTT_PLAN_MFMA: return mfma ? TTT_PLAN_MFMA : TTT_ERR_UNSUPPORTED;
    case TTT_PLAN_BIGCHUNK:
    case TTT_PLAN_SPLIT: return TTT_ERR_UNSUPPORTED;
    default: break;
    }
    return mfma ? TTT_PLAN_MFMA : TTT_PLAN_GENERIC;
}

int launch_status(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_LAUNCH; }

// Workspace of ttt_linear_fwd_noalloc: one static array per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the host
// the name is only a stand-in for the symbol); it passes the device address
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = TTT_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch array (nullptr on failure, with the
// HIP error in *err).
void* scratch_address(int device, hipError_t* err)
{
    std::call_once(g_scratch_once[device], [device] {
        void* p = nullptr;
        g_scratch_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[device] = g_scratch_err[device] == hipSuccess ? p : nullptr;
    });
    *err = g_scratch_err[device];
    return g_scratch_ptr[device];
}

}  // namespace

extern "C" {

const char* ttt_status_string(int status)
{
    switch (status) {
    case TTT_OK: return "ok";
    case TTT_ERR_INVALID_ARG: return "invalid argument";
    case TTT_ERR_UNSUPPORTED: return "unsupported shape, dtype or plan";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    case TTT_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char* ttt_plan_name(int plan)
{
    switch (plan) {
    case TTT_PLAN_AUTO: return "auto";
    case TTT_PLAN_GENERIC: return "generic";
    case TTT_PLAN_MFMA: return "mfma";
    case TTT_PLAN_BIGCHUNK: return "bigchunk";
    case TTT_PLAN_SPLIT: return "split";
    default: return "unknown plan";
    }
}

int ttt_linear_select_plan(int B, int H, int T, int d, int chunk, int io_dtype, int plan)
{
    return linear_plan(B, H, T, d, chunk, io_dtype, plan);
}

int ttt_linear_select_plan_ex(int B, int H, int T, int d, int chunk, int io_dtype, int plan,
                              int read_mode)
{
    return linear_plan(B, H, T, d, chunk, io_dtype, plan, read_mode);
}

size_t ttt_linear_workspace_bytes_ex(int B, int H, int T, int d, int chunk, int io_dtype,
                                     int plan)
{
    int p = linear_plan(B, H, T, d, chunk, io_dtype, plan);
    if (p == TTT_PLAN_BIGCHUNK) return linear_bigchunk_workspace(B * H, T, d, chunk);
    if (p == TTT_PLAN_SPLIT) return linear_seg_workspace(B * H, T, d);
    return 0;
}

// The size-only query: enough for whatever plan either I/O type selects.
size_t ttt_linear_workspace_bytes(int B, int H, int T, int d, int chunk)
{
    size_t n = 0;
    for (int io : {(int)TTT_DTYPE_F32, (int)TTT_DTYPE_BF16})
        for (int plan = TTT_PLAN_AUTO; plan <= TTT_PLAN_SPLIT; ++plan) {
            const size_t m = ttt_linear_workspace_bytes_ex(B, H, T, d, chunk, io, plan);
            n = m > n ? m : n;
        }
    return n;
}

int ttt_linear_fwd(const void* K, const void* Q, const void* V,
                   const float* eta, float eta_scalar, const float* W0,
                   void* Z, float* W_out,
                   int B, int H, int T, int d, int chunk, int io_dtype,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    return ttt_linear_fwd_ex(K, Q, V, eta, eta_scalar, W0, Z, W_out, B, H, T, d, chunk,
                             io_dtype, workspace, workspace_bytes, stream, TTT_PLAN_AUTO,
                             TTT_READ_INCLUSIVE);
}

int ttt_linear_fwd_ex(const void* K, const void* Q, const void* V,
                      const float* eta, float eta_scalar, const float* W0,
                      void* Z, float* W_out,
                      int B, int H, int T, int d, int chunk, int io_dtype,
                      void* workspace, size_t workspace_bytes, void* stream, int plan,
                      int read_mode)
{
    if (!K || !Q || !V || !W0 || !Z || !W_out) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W0, 16) || !aligned(W_out, 16))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    const int p = linear_plan(B, H, T, d, chunk, io_dtype, plan, read_mode);
    if (p < 0) return p;
    const size_t need = ttt_linear_workspace_bytes_ex(B, H, T, d, chunk, io_dtype, p);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return TTT_ERR_WORKSPACE;

    LinearArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar; a.W0 = W0;
    a.Z = Z; a.W_out = W_out; a.BH = B * H; a.T = T; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    a.read_start = read_mode == TTT_READ_CHUNK_START;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.cu = nullptr; a.H = H; a.total_T = T;
    a.momentum = 0; a.beta = 0.f; a.mom0 = nullptr; a.mom_out = nullptr;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (p) {
    case TTT_PLAN_MFMA:
        return launch_status(a.bf16 ? launch_linear_mfma(a, s) : launch_linear_f32(a, s));
    case TTT_PLAN_BIGCHUNK: return launch_status(launch_linear_bigchunk(a, s));
    case TTT_PLAN_SPLIT: return launch_status(launch_linear_seg(a, s));
    default: return launch_status(launch_linear_generic(a, s));
    }
}

int ttt_linear_fwd_noalloc(const void* K, const void* Q, const void* V,
                           const float* eta, float eta_scalar, const float* W0,
                           void* Z, float* W_out,
                           int B, int H, int T, int d, int chunk, int io_dtype, void* stream)
{
    // the same host checks as ttt_linear_fwd, then the workspace size against the
    // static scratch, before any HIP call
    if (!K || !Q || !V || !W0 || !Z || !W_out) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W0, 16) || !aligned(W_out, 16))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    const int p = linear_plan(B, H, T, d, chunk, io_dtype, TTT_PLAN_AUTO);
    if (p < 0) return p;
    const size_t need = ttt_linear_workspace_bytes_ex(B, H, T, d, chunk, io_dtype, p);
    if (need > kScratchBytes) return TTT_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return TTT_ERR_LAUNCH;
        hipError_t err;
        ws = scratch_address(dev, &err);
        if (!ws) return TTT_ERR_LAUNCH;
    }
    return ttt_linear_fwd_ex(K, Q, V, eta, eta_scalar, W0, Z, W_out, B, H, T, d, chunk,
                             io_dtype, ws, ws ? kScratchBytes : 0, stream, p,
                             TTT_READ_INCLUSIVE);
}

size_t ttt_linear_noalloc_scratch_bytes(void) { return kScratchBytes; }

size_t ttt_linear_bwd_workspace_bytes(int B, int H, int T, int d, int chunk, int io_dtype)
{
    if (!dims_ok(B, H, T, d, chunk)) return 0;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return 0;
    if (d != 16 && d != 32 && d != 64 && d != 128) return 0;
    return linear_bwd_workspace(B * H, T, d, chunk, io_dtype == TTT_DTYPE_BF16);
}

int ttt_linear_bwd(const void* K, const void* Q, const void* V,
                   const float* eta, float eta_scalar, const float* W0,
                   const void* dZ, const float* dW_T,
                   void* dK, void* dQ, void* dV, float* deta, float* dW0,
                   int B, int H, int T, int d, int chunk, int io_dtype,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    if (!K || !Q || !V || !W0 || !dZ || !dK || !dQ || !dV || !dW0) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(dZ, 16) ||
        !aligned(W0, 16) || !aligned(dK, 16) || !aligned(dQ, 16) || !aligned(dV, 16) ||
        !aligned(dW0, 16) || (dW_T && !aligned(dW_T, 16)))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    if (deta && !aligned(deta, 4)) return TTT_ERR_INVALID_ARG;
    if (!dims_ok(B, H, T, d, chunk)) return TTT_ERR_INVALID_ARG;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    const size_t need = linear_bwd_workspace(B * H, T, d, chunk, io_dtype == TTT_DTYPE_BF16);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return TTT_ERR_WORKSPACE;

    LinearBwdArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar; a.W0 = W0;
    a.dZ = dZ; a.dW_T = dW_T; a.dK = dK; a.dQ = dQ; a.dV = dV; a.deta = deta; a.dW0 = dW0;
    a.BH = B * H; a.T = T; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return launch_status(launch_linear_bwd(a, reinterpret_cast<hipStream_t>(stream)));
}

int ttt_linear_fwd_momentum(const void* K, const void* Q, const void* V,
                            const float* eta, float eta_scalar, const float* W0,
                            const float* Mom0, float beta,
                            void* Z, float* W_out, float* Mom_out,
                            int B, int H, int T, int d, int chunk, int io_dtype,
                            void* workspace, size_t workspace_bytes, void* stream, int plan)
{
    if (!K || !Q || !V || !W0 || !Z || !W_out || !Mom_out) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W0, 16) || !aligned(W_out, 16) || !aligned(Mom_out, 16) ||
        (Mom0 && !aligned(Mom0, 16)))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    if (!(beta >= 0.f && beta < 1.f)) return TTT_ERR_INVALID_ARG;
    const int p = linear_plan(B, H, T, d, chunk, io_dtype, plan, TTT_READ_CHUNK_START);
    if (p < 0) return p;
    const size_t need = ttt_linear_workspace_bytes_ex(B, H, T, d, chunk, io_dtype, p);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return TTT_ERR_WORKSPACE;

    LinearArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar; a.W0 = W0;
    a.Z = Z; a.W_out = W_out; a.BH = B * H; a.T = T; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    a.read_start = 1;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.cu = nullptr; a.H = H; a.total_T = T;
    a.momentum = 1; a.beta = beta; a.mom0 = Mom0; a.mom_out = Mom_out;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p == TTT_PLAN_BIGCHUNK) return launch_status(launch_linear_bigchunk(a, s));
    return launch_status(launch_linear_generic(a, s));
}

int ttt_linear_ln_fwd(const void* K, const void* Q, const void* V,
                      const float* eta, float eta_scalar, const float* W0, const float* b0,
                      const float* ln_weight, const float* ln_bias, float eps,
                      void* Z, float* W_out, float* b_out,
                      int B, int H, int T, int d, int chunk, int io_dtype, void* stream)
{
    if (!K || !Q || !V || !W0 || !b0 || !Z || !W_out || !b_out) return TTT_ERR_INVALID_ARG;
    if ((ln_weight == nullptr) != (ln_bias == nullptr)) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W0, 16) || !aligned(W_out, 16) || !aligned(b0, 4) || !aligned(b_out, 4) ||
        (ln_weight && (!aligned(ln_weight, 4) || !aligned(ln_bias, 4))))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || !(eps > 0.f)) return TTT_ERR_INVALID_ARG;
    if (!dims_ok(B, H, T, d, chunk)) return TTT_ERR_INVALID_ARG;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;

    LinearLnArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar;
    a.W0 = W0; a.b0 = b0; a.ln_weight = ln_weight; a.ln_bias = ln_bias; a.eps = eps;
    a.Z = Z; a.W_out = W_out; a.b_out = b_out;
    a.BH = B * H; a.H = H; a.T = T; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    return launch_status(launch_linear_ln(a, reinterpret_cast<hipStream_t>(stream)));
}

int ttt_linear_step(const void* K, const void* Q, const void* V,
                    const float* eta, float eta_scalar, float* W_chunk, float* G, int pos,
                    void* Z, int B, int H, int n, int d, int chunk, int io_dtype, void* stream)
{
    if (!K || !Q || !V || !W_chunk || !G || !Z) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W_chunk, 16) || !aligned(G, 16))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    if (!dims_ok(B, H, n, d, chunk)) return TTT_ERR_INVALID_ARG;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARG;
    if (pos < 0 || pos >= chunk) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    // the carried state and its in-chunk update must be disjoint
    const uintptr_t wlo = reinterpret_cast<uintptr_t>(W_chunk), glo = reinterpret_cast<uintptr_t>(G);
    const uintptr_t state_bytes = (uintptr_t)B * H * d * d * sizeof(float);
    if (wlo < glo + state_bytes && glo < wlo + state_bytes) return TTT_ERR_INVALID_ARG;

    LinearArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar; a.W0 = W_chunk;
    a.Z = Z; a.W_out = W_chunk; a.BH = B * H; a.T = n; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    a.read_start = 0;
    a.cu = nullptr; a.H = H; a.total_T = n;
    a.momentum = 0; a.beta = 0.f; a.mom0 = nullptr; a.mom_out = nullptr;
    a.workspace = nullptr; a.workspace_bytes = 0;
    return launch_status(launch_linear_step(a, G, pos, reinterpret_cast<hipStream_t>(stream)));
}

int ttt_linear_select_plan_varlen(int n_docs, int H, int total_T, int d, int chunk,
                                  int io_dtype, int plan)
{
    if (n_docs <= 0 || H <= 0 || total_T < 0 || d <= 0 || chunk <= 0) return TTT_ERR_INVALID_ARG;
    if ((long double)H * ((long double)total_T + 1) * d >= 4.0e18L ||
        (long double)n_docs * H * 64 >= 2.0e9L)
        return TTT_ERR_INVALID_ARG;
    if (io_dtype != TTT_DTYPE_F32 && io_dtype != TTT_DTYPE_BF16) return TTT_ERR_INVALID_ARG;
    if (plan < TTT_PLAN_AUTO || plan > TTT_PLAN_SPLIT) return TTT_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
    const bool mfma = chunk <= 16 && linear_mfma_supported(d, chunk, io_dtype == TTT_DTYPE_BF16);
    switch (plan) {
    case TTT_PLAN_GENERIC: return TTT_PLAN_GENERIC;
    case TTT_PLAN_MFMA: return mfma ? TTT_PLAN_MFMA : TTT_ERR_UNSUPPORTED;
    case TTT_PLAN_BIGCHUNK:
    case TTT_PLAN_SPLIT: return TTT_ERR_UNSUPPORTED;
    default: return mfma ? TTT_PLAN_MFMA : TTT_PLAN_GENERIC;
    }
}

int ttt_linear_fwd_varlen(const void* K, const void* Q, const void* V,
                          const float* eta, float eta_scalar, const float* W0,
                          void* Z, float* W_out, const int* cu_seqlens,
                          int n_docs, int H, int total_T, int d, int chunk, int io_dtype,
                          void* stream, int plan)
{
    if (!K || !Q || !V || !W0 || !Z || !W_out || !cu_seqlens) return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W0, 16) || !aligned(W_out, 16) || !aligned(cu_seqlens, 4))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    const int p = ttt_linear_select_plan_varlen(n_docs, H, total_T, d, chunk, io_dtype, plan);
    if (p < 0) return p;

    LinearArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar; a.W0 = W0;
    a.Z = Z; a.W_out = W_out; a.BH = n_docs * H; a.T = 0; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    a.read_start = 0;
    a.workspace = nullptr; a.workspace_bytes = 0;
    a.cu = cu_seqlens; a.H = H; a.total_T = total_T;
    a.momentum = 0; a.beta = 0.f; a.mom0 = nullptr; a.mom_out = nullptr;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p == TTT_PLAN_MFMA) return launch_status(launch_linear_mfma(a, s));
    return launch_status(launch_linear_generic(a, s));
}

int ttt_mlp_select_plan(int B, int H, int T, int d, int chunk, int io_dtype, int plan)
{
    return mlp_plan(B, H, T, d, chunk, io_dtype, plan);
}

size_t ttt_mlp_workspace_bytes_ex(int B, int H, int T, int d, int chunk, int io_dtype, int plan)
{
    int p = mlp_plan(B, H, T, d, chunk, io_dtype, plan);
    if (p == TTT_PLAN_GENERIC) return mlp_generic_workspace(B * H, T, d, chunk);
    return 0;
}

size_t ttt_mlp_workspace_bytes(int B, int H, int T, int d, int chunk)
{
    size_t n = 0;
    for (int io : {(int)TTT_DTYPE_F32, (int)TTT_DTYPE_BF16})
        for (int plan = TTT_PLAN_AUTO; plan <= TTT_PLAN_SPLIT; ++plan) {
            const size_t m = ttt_mlp_workspace_bytes_ex(B, H, T, d, chunk, io, plan);
            n = m > n ? m : n;
        }
    return n;
}

int ttt_mlp_fwd(const void* K, const void* Q, const void* V,
                const float* eta, float eta_scalar,
                const float* W1_0, const float* b1_0, const float* W2_0, const float* b2_0,
                void* Z, float* W1_out, float* b1_out, float* W2_out, float* b2_out,
                int B, int H, int T, int d, int chunk, int io_dtype,
                void* workspace, size_t workspace_bytes, void* stream)
{
    return ttt_mlp_fwd_ex(K, Q, V, eta, eta_scalar, W1_0, b1_0, W2_0, b2_0, Z, W1_out, b1_out,
                          W2_out, b2_out, B, H, T, d, chunk, io_dtype, workspace,
                          workspace_bytes, stream, TTT_PLAN_AUTO);
}

int ttt_mlp_fwd_ex(const void* K, const void* Q, const void* V,
                   const float* eta, float eta_scalar,
                   const float* W1_0, const float* b1_0, const float* W2_0, const float* b2_0,
                   void* Z, float* W1_out, float* b1_out, float* W2_out, float* b2_out,
                   int B, int H, int T, int d, int chunk, int io_dtype,
                   void* workspace, size_t workspace_bytes, void* stream, int plan)
{
    if (!K || !Q || !V || !W1_0 || !W2_0 || !Z || !W1_out || !W2_out) return TTT_ERR_INVALID_ARG;
    if ((b1_0 == nullptr) != (b1_out == nullptr) || (b2_0 == nullptr) != (b2_out == nullptr))
        return TTT_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Q, 16) || !aligned(V, 16) || !aligned(Z, 16) ||
        !aligned(W1_0, 16) || !aligned(W2_0, 16) || !aligned(W1_out, 16) ||
        !aligned(W2_out, 16))
        return TTT_ERR_INVALID_ARG;
    if ((b1_0 && (!aligned(b1_0, 4) || !aligned(b1_out, 4))) ||
        (b2_0 && (!aligned(b2_0, 4) || !aligned(b2_out, 4))))
        return TTT_ERR_INVALID_ARG;
    if (eta ? !aligned(eta, 4) : !std::isfinite(eta_scalar)) return TTT_ERR_INVALID_ARG;
    const int p = mlp_plan(B, H, T, d, chunk, io_dtype, plan);
    if (p < 0) return p;
    const size_t need = ttt_mlp_workspace_bytes_ex(B, H, T, d, chunk, io_dtype, p);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return TTT_ERR_WORKSPACE;

    MlpArgs a;
    a.K = K; a.Q = Q; a.V = V; a.eta = eta; a.eta_scalar = eta_scalar;
    a.W1 = W1_0; a.b1 = b1_0; a.W2 = W2_0; a.b2 = b2_0;
    a.Z = Z; a.W1_out = W1_out; a.b1_out = b1_out; a.W2_out = W2_out; a.b2_out = b2_out;
    a.BH = B * H; a.T = T; a.d = d; a.chunk = chunk;
    a.bf16 = io_dtype == TTT_DTYPE_BF16;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p == TTT_PLAN_MFMA) return launch_status(launch_mlp_mfma(a, s));
    return launch_status(launch_mlp_generic(a, s));
}

}  // extern "C"
