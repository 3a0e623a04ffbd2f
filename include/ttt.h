/*
 * ttt.h — C ABI of libttt_amd.so: forward scan of a test-time-training (TTT)
 * layer on an AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A TTT layer carries, per (batch, head), a fast-weight state that is itself a
 * small model; reading the sequence trains that model one gradient step at a
 * time (PaperTrace "5 · TestingTime 训练与长上下文" §1.1 and §2.1: an initial
 * state W0, an update rule W_t = W_{t-1} - eta * grad l(W_{t-1}; x_t) and an
 * output rule y_t = f(q_t; W_t); keys, queries and values arrive already
 * projected).  The loss is the key-to-value reconstruction
 * l = 1/2 ||f(k_t) - v_t||^2 (same page §2.3).  Tokens are taken in chunks of
 * `chunk` tokens (same page §1.1, "b = 16"); every gradient in a chunk is taken
 * at the chunk-start state, token t reads with the chunk's updates up to and
 * including its own, and the state then advances by the eta-weighted sum of the
 * chunk's gradients.  eta_s scales the gradient of token s (the writer).
 *
 *   TTT-Linear  f_W(k) = W k,               W  : d x d            (§2.3)
 *   TTT-MLP     f(k) = W2 gelu(W1 k + b1) + b2, W1 : 4d x d, b1 : 4d,
 *               W2 : d x 4d, b2 : d; GELU in its exact erf form
 *               (diosapp "Test-Time Training (TTT) guide" §3: two layers,
 *               hidden width 4x, GELU)
 *
 * Inside a chunk the kernels use the dual form (diosapp guide §3; PaperTrace
 * §1.1): for TTT-Linear, with the chunk's keys/queries/values as columns,
 *   E = W K - V,   Z = W Q - E diag(eta) triu(K^T Q),   W <- W - E diag(eta) K^T.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous.
 *    K, Q, V, Z, W0/W_out, W1/W2 and their outputs must be 16-byte aligned;
 *    eta and the bias vectors 4-byte aligned.
 *  - K, Q, V  : [B, H, T, d] in `io_dtype` (one row of d features per token).
 *    Z        : [B, H, T, d] in `io_dtype` (fp32 -> bf16 rounds to nearest even).
 *    eta      : [B, H, T] fp32 per-token learning rate, or NULL to use
 *               `eta_scalar` for every token.
 *    states   : always fp32; row index = output feature.
 *  - Any T >= 1; a last chunk shorter than `chunk` is processed with the
 *    tokens it has.
 *  - Ownership: the caller allocates every buffer, including the workspace.
 *    The library allocates no device memory, keeps no state between calls and
 *    may be called from several host threads at once.
 *  - Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream).  It is declared `void*` so that this header compiles
 *    without the HIP headers; the calling convention is that of the pointer
 *    hipStream_t is.  The call returns before the work completes; outputs are
 *    valid once the stream has been synchronised.  The library never
 *    synchronises.
 *  - `io_dtype` and `plan` take the ttt_dtype and ttt_plan values (passed as
 *    int, the enums' own calling convention).
 *  - Aliasing: the final-state outputs may alias the matching initial-state
 *    inputs (W_out == W0 updates in place).  Z must not overlap any input.
 *  - Errors: arguments are checked on the host before any HIP call; a failed
 *    check returns a negative ttt_status and enqueues nothing.  A kernel
 *    launch failure returns TTT_ERR_LAUNCH.  Non-finite values inside tensors
 *    are not checked: they propagate (IEEE) within their own (batch, head)
 *    slice only.
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TTT_OK = 0,
    TTT_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, non-positive size, bad enum,
                                   non-finite eta_scalar with eta == NULL */
    TTT_ERR_UNSUPPORTED = -2,   /* valid arguments outside what the kernels implement */
    TTT_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
    TTT_ERR_LAUNCH = -4         /* the HIP runtime rejected a kernel launch */
} ttt_status;

typedef enum {
    TTT_DTYPE_F32 = 0,          /* K, Q, V, Z in fp32 */
    TTT_DTYPE_BF16 = 1          /* K, Q, V, Z in bf16; arithmetic accumulates in fp32 */
} ttt_dtype;

/* Kernel plans.  AUTO picks the fastest plan that supports the shape; the others
 * force one (TTT_ERR_UNSUPPORTED if it cannot run the shape) so that tests can
 * compare plans on the same inputs. */
typedef enum {
    TTT_PLAN_AUTO = 0,
    TTT_PLAN_GENERIC = 1,       /* fp32 vector ALU, any chunk, fp32 or bf16 I/O */
    TTT_PLAN_MFMA = 2,          /* matrix cores, inclusive read.  bf16 I/O: bf16 matrix
                                   cores, d in {32, 64, 128}, chunk <= 16 or a multiple
                                   of 16.  fp32 I/O: fp32 matrix cores, d in {16, 32,
                                   64, 128}, any chunk (not for packed documents) */
    TTT_PLAN_BIGCHUNK = 3,      /* bf16 matrix cores, three stages, d in {64, 128}, chunk a
                                   multiple of 32 >= 128 */
    TTT_PLAN_SPLIT = 4          /* bf16 matrix cores, inclusive read, d = 64, chunk 16,
                                   T >= 2048, at most 64 (batch, head) slices (AUTO
                                   takes it up to 32 slices, and from 33 to 64 when
                                   T >= 4096): each sequence in S ~ 256 / slices + 1
                                   segments; segment 0 scans while segments 1 .. S-2
                                   form their affine maps, a combine gives every
                                   segment its start state, and segments 1 .. S-1
                                   scan again from it (workspace: 3 S d^2 fp32 per
                                   slice) */
} ttt_plan;

/* Read order of a chunk's tokens.  INCLUSIVE: token t reads with the chunk's
 * updates up to and including its own (the dual form above).  CHUNK_START:
 * every token of a chunk reads with the chunk-start state, z_t = W_c q_t (apply,
 * then update: the large-chunk ordering that leaves in-chunk dependencies to
 * window attention, PaperTrace "5 · TestingTime 训练与长上下文" §1.1, and the
 * read/write-order passage of its §2.4; with chunk == 1 the read-before-write
 * delta rule).  The state update is the same in both. */
typedef enum {
    TTT_READ_INCLUSIVE = 0,
    TTT_READ_CHUNK_START = 1
} ttt_read_mode;

/* ------------------------------------------------------------------------ */
/* TTT-Linear                                                                */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace ttt_linear_fwd needs for this shape: the largest size any
 * plan needs for either I/O dtype (0 when none does).  A workspace of this size
 * serves ttt_linear_fwd and ttt_linear_fwd_ex for the shape whatever their
 * dtype and plan. */
size_t ttt_linear_workspace_bytes(int B, int H, int T, int d, int chunk);

/* Bytes of workspace for this shape, dtype and plan exactly (0 when none, and
 * for shapes the plan cannot run). */
size_t ttt_linear_workspace_bytes_ex(int B, int H, int T, int d, int chunk,
                                     int io_dtype, int plan);

/* Plan that ttt_linear_fwd would run for this shape (never TTT_PLAN_AUTO), or a
 * negative ttt_status if no plan supports it. */
int ttt_linear_select_plan(int B, int H, int T, int d, int chunk, int io_dtype, int plan);

/* Forward scan of TTT-Linear (plan AUTO, inclusive read).
 *   W0    : [B, H, d, d] fp32 initial state.
 *   W_out : [B, H, d, d] fp32 state after the last token (may alias W0).
 *   d     : 16, 32, 64 or 128.   chunk : >= 1.
 *   workspace / workspace_bytes : device scratch of at least
 *           ttt_linear_workspace_bytes_ex(..., io_dtype, TTT_PLAN_AUTO) bytes
 *           (ttt_linear_workspace_bytes(...) always suffices), 256-byte aligned
 *           (may be NULL when that is 0).
 * The state update follows PaperTrace "5 · TestingTime 训练与长上下文" §1.1/§2.3;
 * with chunk == 1 it is the delta rule of the same page §2.1. */
int ttt_linear_fwd(const void* K, const void* Q, const void* V,
                   const float* eta, float eta_scalar,
                   const float* W0,
                   void* Z, float* W_out,
                   int B, int H, int T, int d, int chunk, int io_dtype,
                   void* workspace, size_t workspace_bytes,
                   void* stream);

/* TTT-Linear with a momentum state (the E2-TTT passage of "Test-Time Training
 * (TTT)", §2.3 and §5.1: fast weights and a momentum evolve per chunk from the
 * gradient at the chunk start).  With grad_c the eta-weighted sum of chunk c's
 * token gradients at its start state W_c:
 *   Mom_{c+1} = beta Mom_c + (1 - beta) grad_c,   W_{c+1} = W_c - Mom_{c+1},
 * and every token of a chunk reads with W_c (z_t = W_c q_t), as the passage
 * states the update per chunk only.  beta = 0 is ttt_linear_fwd_ex with
 * TTT_READ_CHUNK_START.
 *   Mom0     : [B, H, d, d] fp32 initial momentum, or NULL for zero.
 *   Mom_out  : [B, H, d, d] fp32 final momentum (may alias Mom0).
 *   beta     : 0 <= beta < 1.
 *   Plans: GENERIC (any chunk) and BIGCHUNK (as ttt_linear_fwd; its workspace);
 *   MFMA is TTT_ERR_UNSUPPORTED.  Other arguments as ttt_linear_fwd. */
int ttt_linear_fwd_momentum(const void* K, const void* Q, const void* V,
                            const float* eta, float eta_scalar, const float* W0,
                            const float* Mom0, float beta,
                            void* Z, float* W_out, float* Mom_out,
                            int B, int H, int T, int d, int chunk, int io_dtype,
                            void* workspace, size_t workspace_bytes, void* stream, int plan);

/* TTT-Linear with the inner bias as part of the state and, when ln_weight is
 * given, LayerNorm and a residual inside the inner model:
 *   f(x) = x + LN(W x + b),  LN(u) = ln_weight * (u - mean(u)) / sqrt(var(u) + eps)
 *                                    + ln_bias   (over the d features),
 * or f(x) = W x + b when ln_weight == ln_bias == NULL (diosapp "Test-Time
 * Training (TTT) guide" §3 gives f(x) = W x + b; the LN-and-residual ablation
 * is the one of PaperTrace "5 · TestingTime 训练与长上下文" §3.1).  W and b
 * take the chunked gradient step of ttt_linear_fwd (loss 1/2 ||f(k) - v||^2,
 * gradients at the chunk-start state, inclusive read); ln_weight and ln_bias
 * are fixed (outer-model parameters).
 *   b0, b_out            : [B, H, d] fp32 (b_out may alias b0; b0 may be zeros).
 *   ln_weight, ln_bias   : [H, d] fp32, shared by the batch, or both NULL.
 *   eps                  : > 0, finite.
 *   Others as ttt_linear_fwd; d : 16, 32, 64 or 128; any chunk; fp32 arithmetic
 *   on the fp32 matrix cores, one workgroup per (batch, head); no workspace. */
int ttt_linear_ln_fwd(const void* K, const void* Q, const void* V,
                      const float* eta, float eta_scalar, const float* W0, const float* b0,
                      const float* ln_weight, const float* ln_bias, float eps,
                      void* Z, float* W_out, float* b_out,
                      int B, int H, int T, int d, int chunk, int io_dtype, void* stream);

/* Packed documents with a reset at every document (variable-length batches).
 * Each document of every head is its own TTT-Linear scan from its own initial
 * state: no state, gradient or output crosses a document boundary, and chunks
 * are counted from the document's first token (PaperTrace "5 · TestingTime
 * 训练与长上下文" §2.4, the cross-sequence reset passage: each independent
 * document needs its own W0 and state).
 *   K, Q, V, Z  : [H, total_T, d] in io_dtype, head-major: document n of head h is
 *                 rows cu_seqlens[n] .. cu_seqlens[n+1]-1 of head h's block.
 *   eta         : [H, total_T] fp32 or NULL (eta_scalar).
 *   W0, W_out   : [n_docs, H, d, d] fp32 (W_out may alias W0).
 *   cu_seqlens  : DEVICE int32 [n_docs + 1], non-decreasing offsets into
 *                 [0, total_T] (read on the GPU; values outside are clamped, so a
 *                 malformed table gives wrong documents, never an out-of-range
 *                 access).  An empty document passes W0 through.  Rows that no
 *                 document covers are not written in Z.
 *   d : 16, 32, 64 or 128;  chunk >= 1;  plans: GENERIC, and MFMA for bf16 with
 *   chunk <= 16 (AUTO picks it); no workspace. */
int ttt_linear_fwd_varlen(const void* K, const void* Q, const void* V,
                          const float* eta, float eta_scalar, const float* W0,
                          void* Z, float* W_out, const int* cu_seqlens,
                          int n_docs, int H, int total_T, int d, int chunk, int io_dtype,
                          void* stream, int plan);

/* Plan that ttt_linear_fwd_varlen would run (never TTT_PLAN_AUTO), or a negative
 * ttt_status. */
int ttt_linear_select_plan_varlen(int n_docs, int H, int total_T, int d, int chunk,
                                  int io_dtype, int plan);

/* Bytes of workspace ttt_linear_bwd needs: the chunk-start states
 * (B*H*(ceil(T/chunk)+1)*d*d fp32) and one fp32 plane of dK, dQ and deta per
 * 16-row block of the state ((d/16)*B*H*T*(2d+1) fp32), each piece rounded up
 * to 256 bytes; the same for either I/O type.  0 for an unsupported shape. */
size_t ttt_linear_bwd_workspace_bytes(int B, int H, int T, int d, int chunk, int io_dtype);

/* Backward pass (vector-Jacobian product) of ttt_linear_fwd: for the scalar
 * L = <dZ, Z> + <dW_T, W_out> it writes the gradients with respect to K, Q, V,
 * each token's eta and W0.  The forward scan is recomputed from W0 (nothing is
 * kept from a ttt_linear_fwd call).  Same chunking and semantics as
 * ttt_linear_fwd (PaperTrace "5 · TestingTime 训练与长上下文" §1.1, §2.1, §2.3).
 *   K, Q, V, dZ    : [B, H, T, d] in io_dtype (dZ: the cotangent of Z).
 *   eta            : [B, H, T] fp32 or NULL (eta_scalar for every token).
 *   W0             : [B, H, d, d] fp32.
 *   dW_T           : [B, H, d, d] fp32 cotangent of W_out, or NULL for zero.
 *   dK, dQ, dV     : [B, H, T, d] in io_dtype (outputs).
 *   deta           : [B, H, T] fp32, the gradient for each token's eta (also
 *                    when eta is NULL: the gradient of eta_scalar is then the
 *                    sum of deta), or NULL to skip it.
 *   dW0            : [B, H, d, d] fp32 (output).
 *   d : 16, 32, 64 or 128;  chunk >= 1.
 *   workspace      : at least ttt_linear_bwd_workspace_bytes(...) bytes,
 *                    256-byte aligned.
 * Arithmetic is fp32 (inputs in bf16 are widened exactly).  dK, dQ and deta
 * are sums over the state's 16-row blocks, each block's terms kept in its own
 * fp32 plane of the workspace and the planes added in a fixed order: every
 * output is the same bits on every call.  Outputs must not overlap inputs or
 * each other. */
int ttt_linear_bwd(const void* K, const void* Q, const void* V,
                   const float* eta, float eta_scalar, const float* W0,
                   const void* dZ, const float* dW_T,
                   void* dK, void* dQ, void* dV, float* deta, float* dW0,
                   int B, int H, int T, int d, int chunk, int io_dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Streaming continuation of the TTT-Linear scan: n more tokens of every
 * (batch, head) sequence, from a carried state, with the same chunking as
 * ttt_linear_fwd over the whole sequence (token i of the sequence belongs to
 * chunk floor(i / chunk)).  Inside a chunk every gradient is taken at the
 * chunk-start state and a token reads with the chunk's updates up to and
 * including its own (PaperTrace "5 · TestingTime 训练与长上下文" §1.1, §2.1,
 * §2.3), so the carried state is a pair:
 *   W_chunk : [B, H, d, d] fp32, the state at the start of the current chunk;
 *   G       : [B, H, d, d] fp32, the sum over the chunk's tokens so far of
 *             eta_s (W_chunk k_s - v_s) k_s^T;
 *   pos     : how many tokens of the current chunk came before this call,
 *             0 <= pos < chunk (the caller tracks it: after the call it is
 *             (pos + n) % chunk).
 * The state after the last token read so far is W_chunk - G.  Both are updated
 * in place; when a chunk completes W_chunk becomes W_chunk - G and G is zeroed.
 * A stream starts from W_chunk = W0, G = 0, pos = 0; ttt_linear_fwd over a
 * prefix whose length is a multiple of chunk hands over W_out with G = 0.
 *   K, Q, V : [B, H, n, d] in io_dtype;  eta : [B, H, n] fp32 or NULL;
 *   Z       : [B, H, n, d] in io_dtype;  d : 16, 32, 64 or 128;  n >= 1.
 * W_chunk and G must not overlap each other or any other argument.  Arithmetic
 * is fp32 on the vector ALUs; no workspace. */
int ttt_linear_step(const void* K, const void* Q, const void* V,
                    const float* eta, float eta_scalar,
                    float* W_chunk, float* G, int pos,
                    void* Z, int B, int H, int n, int d, int chunk, int io_dtype,
                    void* stream);

/* ttt_linear_fwd with a kernel plan (ttt_plan) and a choice of read order
 * (ttt_read_mode); ttt_linear_fwd is this call with TTT_PLAN_AUTO and
 * TTT_READ_INCLUSIVE.  CHUNK_START runs on the GENERIC and BIGCHUNK plans (MFMA:
 * TTT_ERR_UNSUPPORTED); an unknown read_mode is TTT_ERR_INVALID_ARG.  Workspace
 * sizes are those of ttt_linear_workspace_bytes_ex for the plan that runs. */
int ttt_linear_fwd_ex(const void* K, const void* Q, const void* V,
                      const float* eta, float eta_scalar,
                      const float* W0,
                      void* Z, float* W_out,
                      int B, int H, int T, int d, int chunk, int io_dtype,
                      void* workspace, size_t workspace_bytes,
                      void* stream, int plan, int read_mode);

/* ttt_linear_fwd for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments as ttt_linear_fwd without the workspace: the plans
 * that need one (TTT_PLAN_BIGCHUNK for chunks of 128+ tokens, TTT_PLAN_SPLIT for
 * a few long chunk-16 heads, at most 12 MiB) run in a static device array of the
 * library, TTT_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU.  The array is part of the
 * library's code object: each GPU holds it from the library's first use there
 * until the process ends.  The call allocates nothing and frees nothing.
 *   - Shapes whose workspace (ttt_linear_workspace_bytes_ex for the AUTO plan)
 *     exceeds 64 MiB return TTT_ERR_WORKSPACE before any HIP call (for example
 *     16 heads x 131072 tokens at d = 128, chunk 2048, which needs 160 MiB: use
 *     ttt_linear_fwd with a caller workspace there).
 *   - The scratch of the caller's current device is used; `stream` must belong
 *     to that device.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in time
 *     on one GPU (other streams, other host threads) race and give wrong
 *     results.  Calls serialised on one stream are safe; each call writes every
 *     scratch byte it reads, so nothing depends on what an earlier call left.
 *   - A failure to find the array's device address returns TTT_ERR_LAUNCH. */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ttt_linear_fwd_noalloc(const void* K, const void* Q, const void* V,
                           const float* eta, float eta_scalar,
                           const float* W0,
                           void* Z, float* W_out,
                           int B, int H, int T, int d, int chunk, int io_dtype,
                           void* stream);

/* Size in bytes of ttt_linear_fwd_noalloc's per-GPU scratch array. */
size_t ttt_linear_noalloc_scratch_bytes(void);

/* Plan that ttt_linear_fwd_ex would run for this shape and read order. */
int ttt_linear_select_plan_ex(int B, int H, int T, int d, int chunk, int io_dtype, int plan,
                              int read_mode);

/* ------------------------------------------------------------------------ */
/* TTT-MLP (hidden width 4d)                                                 */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace ttt_mlp_fwd needs for this shape: the largest size any plan
 * needs for either I/O dtype (0 when none does). */
size_t ttt_mlp_workspace_bytes(int B, int H, int T, int d, int chunk);

/* Bytes of workspace for this shape, dtype and plan exactly. */
size_t ttt_mlp_workspace_bytes_ex(int B, int H, int T, int d, int chunk, int io_dtype, int plan);

int ttt_mlp_select_plan(int B, int H, int T, int d, int chunk, int io_dtype, int plan);

/* Forward scan of TTT-MLP, f(k) = W2 gelu(W1 k + b1) + b2 (plan AUTO).
 *   W1_0 : [B, H, 4d, d]   b1_0 : [B, H, 4d] or NULL (model without b1)
 *   W2_0 : [B, H, d, 4d]   b2_0 : [B, H, d]  or NULL (model without b2)
 *   W1_out, W2_out : final states (may alias W1_0, W2_0);
 *   b1_out / b2_out: final biases, NULL exactly when b1_0 / b2_0 is NULL.
 *   d : 16, 32 or 64 (hidden 4d).  chunk : >= 1.
 *   workspace : at least ttt_mlp_workspace_bytes(...) bytes, 256-byte aligned.
 * A present bias is part of the state and takes the same gradient step; an
 * absent one is a model without that bias.
 * Operand range of the matrix-core plan (bf16 I/O, d = 64, chunk <= 16, which
 * AUTO picks): its products take fp16 operands with fp32 accumulation.  The fp16
 * operands are K, Q, the states W1 and W2, the activations gelu(W1 k + b1), the
 * prediction error E = f(k) - v, the eta-scaled gradients eta E and
 * eta (W2^T E) * gelu', and the token scores k_s . q_t.  Each of them must stay
 * below 65504 in magnitude: past it the operand overflows and the outputs turn
 * non-finite.  Values of at least 2^-14 keep their bf16 value exactly; smaller
 * ones are rounded to fp16's subnormal spacing of 2^-24 (so a tiny eta with a
 * tiny error loses precision).  For data outside that range, call ttt_mlp_fwd_ex
 * with TTT_PLAN_GENERIC (fp32 vector ALU, any magnitude). */
int ttt_mlp_fwd(const void* K, const void* Q, const void* V,
                const float* eta, float eta_scalar,
                const float* W1_0, const float* b1_0,
                const float* W2_0, const float* b2_0,
                void* Z, float* W1_out, float* b1_out, float* W2_out, float* b2_out,
                int B, int H, int T, int d, int chunk, int io_dtype,
                void* workspace, size_t workspace_bytes,
                void* stream);

/* ttt_mlp_fwd with a kernel plan (ttt_plan); the workspace is
 * ttt_mlp_workspace_bytes_ex for the plan that runs. */
int ttt_mlp_fwd_ex(const void* K, const void* Q, const void* V,
                   const float* eta, float eta_scalar,
                   const float* W1_0, const float* b1_0,
                   const float* W2_0, const float* b2_0,
                   void* Z, float* W1_out, float* b1_out, float* W2_out, float* b2_out,
                   int B, int H, int T, int d, int chunk, int io_dtype,
                   void* workspace, size_t workspace_bytes,
                   void* stream, int plan);

/* Static string for a ttt_status value (or "unknown status"). */
const char* ttt_status_string(int status);

/* Static string naming a plan ("generic", "mfma", "bigchunk", ...). */
const char* ttt_plan_name(int plan);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H */
