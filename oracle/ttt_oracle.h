/*
 * ttt_oracle.h — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow fp64 CPU reference for the forward scan of a test-time-training
 * (TTT) layer, and for the gradient of the TTT-Linear scan.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may call it; the product library never links or loads it, and it
 * shares no code, header or constant with the HIP path.
 *
 * Method (sources are the pages the build follows):
 *   - PaperTrace "5 · TestingTime 训练与长上下文" §1.1: a TTT layer is an initial
 *     state W0, an update rule and an output rule; K/Q/V are already projected;
 *     the sequence is cut into chunks of b tokens and every gradient inside a
 *     chunk is taken at the chunk-start state; the output uses the updated model.
 *   - same page §2.1: write W_t = W_{t-1} - eta * grad l(W_{t-1}; x_t),
 *     read y_t = f(q_t; W_t).
 *   - same page §2.3: f_W(k) = W k, l = 1/2 ||W k - v||^2, gradient (W k - v) k^T.
 *   - diosapp "Test-Time Training (TTT) guide" §3: TTT-MLP is a two-layer MLP
 *     with a hidden width of 4x the input and a GELU activation.
 *
 * Readings where the pages leave a step open (each is listed in the design notes):
 *   - loss constant 1/2 (gradient e k^T, no factor 2);
 *   - the chunk update is the eta-weighted SUM of the per-token gradients;
 *   - token t reads with every in-chunk update up to and including its own
 *     (ttt_oracle_linear_read also offers the chunk-start read, the
 *     apply-then-update order of large-chunk TTT: PaperTrace "5 · TestingTime
 *     训练与长上下文" §1.1, and the read/write-order passage of its §2.4);
 *   - eta_t belongs to the writing token (it scales token t's gradient);
 *   - TTT-Linear has no bias; TTT-MLP biases b1, b2 are part of the state and
 *     are updated by the same step, or are absent (frozen zero) when NULL;
 *   - GELU is the exact erf form;
 *   - a final chunk shorter than b is processed with the tokens it has.
 *
 * Layouts (all fp64, row-major, contiguous):
 *   K, Q, V, Z  : [BH, T, d]        one row per token
 *   eta         : [BH, T] or NULL   (NULL -> eta_scalar for every token)
 *   W0, W_out   : [BH, d, d]        row index = output feature
 *   W1          : [BH, hidden, d]   b1 : [BH, hidden]
 *   W2          : [BH, d, hidden]   b2 : [BH, d]
 * Each of the BH (batch, head) slices is independent; `nthreads` worker threads
 * take whole slices (0 -> one per online CPU).  Output buffers must not alias
 * inputs.  Returns the number of threads used (>0) or -1 on a bad argument.
 */
#ifndef TTT_ORACLE_H
#define TTT_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

int ttt_oracle_linear(const double* K, const double* Q, const double* V,
                      const double* eta, double eta_scalar, const double* W0,
                      double* Z, double* W_out,
                      int BH, int T, int d, int chunk, int nthreads);

/* The same scan with a choice of read order: read_start = 0 is the inclusive
 * read above (z_t = (W_c - G_t) q_t); read_start = 1 reads every token of a
 * chunk with the chunk-start state (z_t = W_c q_t: apply, then update).  The
 * state update is the same in both. */
int ttt_oracle_linear_read(const double* K, const double* Q, const double* V,
                           const double* eta, double eta_scalar, const double* W0,
                           double* Z, double* W_out,
                           int BH, int T, int d, int chunk, int read_start, int nthreads);

/* TTT-Linear with the inner bias as state and, when ln_weight is given,
 * LayerNorm and a residual inside f: f(x) = x + LN(W x + b), LN(u) =
 * ln_weight * (u - mean) / sqrt(var + eps) + ln_bias over the d features
 * (ln_weight, ln_bias fixed).  ln_weight == ln_bias == NULL: f(x) = W x + b.
 *   b0, b_out           : [BH, d]
 *   ln_weight, ln_bias  : [BH, d] or both NULL
 * Same chunking, read order and eta conventions as ttt_oracle_linear. */
int ttt_oracle_linear_ln(const double* K, const double* Q, const double* V,
                         const double* eta, double eta_scalar,
                         const double* W0, const double* b0,
                         const double* ln_weight, const double* ln_bias, double eps,
                         double* Z, double* W_out, double* b_out,
                         int BH, int T, int d, int chunk, int nthreads);

/* TTT-Linear with a momentum state M: per chunk, with grad_c the eta-weighted
 * sum of the chunk's token gradients at the chunk-start state,
 * M_{c+1} = beta M_c + (1 - beta) grad_c and W_{c+1} = W_c - M_{c+1}; every
 * token reads with its chunk-start state (z_t = W_c q_t).  M0 may be NULL
 * (zero); 0 <= beta < 1.  M_out : [BH, d, d]. */
int ttt_oracle_linear_momentum(const double* K, const double* Q, const double* V,
                               const double* eta, double eta_scalar, const double* W0,
                               const double* M0, double beta,
                               double* Z, double* W_out, double* M_out,
                               int BH, int T, int d, int chunk, int nthreads);

/* Vector-Jacobian product of ttt_oracle_linear: for L = <dZ, Z> + <dW_T, W_T>
 * (dW_T may be NULL for zero), writes dK, dQ, dV : [BH, T, d], deta : [BH, T]
 * (the gradient for each token's eta, also when eta is NULL and eta_scalar
 * serves every token) and dW0 : [BH, d, d]. */
int ttt_oracle_linear_bwd(const double* K, const double* Q, const double* V,
                          const double* eta, double eta_scalar, const double* W0,
                          const double* dZ, const double* dW_T,
                          double* dK, double* dQ, double* dV, double* deta, double* dW0,
                          int BH, int T, int d, int chunk, int nthreads);

int ttt_oracle_mlp(const double* K, const double* Q, const double* V,
                   const double* eta, double eta_scalar,
                   const double* W1, const double* b1,
                   const double* W2, const double* b2,
                   double* Z, double* W1_out, double* b1_out,
                   double* W2_out, double* b2_out,
                   int BH, int T, int d, int hidden, int chunk, int nthreads);

/* GELU (exact erf form) and its derivative, as the MLP oracle uses them. */
double ttt_oracle_gelu(double x);
double ttt_oracle_gelu_prime(double x);

#ifdef __cplusplus
}
#endif
#endif
