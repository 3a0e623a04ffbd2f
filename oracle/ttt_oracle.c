/*
 * ttt_oracle.c — TEST INFRASTRUCTURE ONLY (see ttt_oracle.h).
 *
 * Per-token primal form of the chunked TTT scan, in fp64, written straight from
 * the definition: for every token the gradient of 1/2||f(k_t) - v_t||^2 is taken
 * at the chunk-start parameters, accumulated with its own eta, and the token's
 * output is read from (chunk-start parameters - accumulated update).  No dual
 * form, no blocking, no fusion.  Threads only split the independent
 * (batch, head) slices.
 */
#include "ttt_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* TTT-Linear, one (batch, head) slice.                                      */
/* PaperTrace "5 · TestingTime 训练与长上下文" §1.1 (chunked update, gradient at */
/* the chunk start, read with the updated model), §2.1 (write/read rules),   */
/* §2.3 (f_W(k) = W k, l = 1/2||W k - v||^2, gradient (W k - v) k^T).        */
/* ------------------------------------------------------------------------ */
static void linear_slice(const double* K, const double* Q, const double* V,
                         const double* eta, double eta_scalar, const double* W0,
                         double* Z, double* W_out, int T, int d, int chunk, int read_start)
{
    double* W  = (double*)malloc(sizeof(double) * d * d);  /* running state      */
    double* Ws = (double*)malloc(sizeof(double) * d * d);  /* chunk-start state  */
    double* G  = (double*)malloc(sizeof(double) * d * d);  /* sum eta_s e_s k_s^T */
    double* e  = (double*)malloc(sizeof(double) * d);
    memcpy(W, W0, sizeof(double) * d * d);

    for (int c0 = 0; c0 < T; c0 += chunk) {
        int c1 = c0 + chunk < T ? c0 + chunk : T;
        memcpy(Ws, W, sizeof(double) * d * d);
        memset(G, 0, sizeof(double) * d * d);
        for (int t = c0; t < c1; ++t) {
            const double* k = K + (size_t)t * d;
            const double* q = Q + (size_t)t * d;
            const double* v = V + (size_t)t * d;
            double et = eta ? eta[t] : eta_scalar;
            /* e_t = Ws k_t - v_t : the loss gradient is e_t k_t^T at Ws */
            for (int i = 0; i < d; ++i) {
                double s = 0.0;
                for (int j = 0; j < d; ++j) s += Ws[i * d + j] * k[j];
                e[i] = s - v[i];
            }
            /* G += eta_t e_t k_t^T  (eta of the writing token) */
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) G[i * d + j] += et * e[i] * k[j];
            /* z_t = (Ws - G) q_t : own update included.  The other read order
             * reads every token of the chunk with the chunk-start state:
             * z_t = Ws q_t (apply, then update). */
            double* z = Z + (size_t)t * d;
            for (int i = 0; i < d; ++i) {
                double s = 0.0;
                if (read_start)
                    for (int j = 0; j < d; ++j) s += Ws[i * d + j] * q[j];
                else
                    for (int j = 0; j < d; ++j) s += (Ws[i * d + j] - G[i * d + j]) * q[j];
                z[i] = s;
            }
        }
        for (int i = 0; i < d * d; ++i) W[i] = Ws[i] - G[i];
    }
    memcpy(W_out, W, sizeof(double) * d * d);
    free(W); free(Ws); free(G); free(e);
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear with a momentum state, one slice.  The E2-TTT passage of        */
/* "Test-Time Training (TTT)" (§2.3, §5.1) keeps a momentum M next to the     */
/* fast weights, updated per chunk from the chunk's gradient at the chunk     */
/* start, M_{c+1} = beta M_c + (1 - beta) grad_c; the step it applies is read  */
/* here as W_{c+1} = W_c - M_{c+1}, with grad_c the eta-weighted sum of the   */
/* chunk's token gradients.  The pages give momentum at chunk level only, so  */
/* every token reads with the chunk-start state: z_t = W_c q_t.  beta = 0 is   */
/* the chunk-start scan.                                                     */
/* ------------------------------------------------------------------------ */
static void linear_momentum_slice(const double* K, const double* Q, const double* V,
                                  const double* eta, double eta_scalar, const double* W0,
                                  const double* M0, double beta, double* Z, double* W_out,
                                  double* M_out, int T, int d, int chunk)
{
    double* W   = (double*)malloc(sizeof(double) * d * d);
    double* Mom = (double*)malloc(sizeof(double) * d * d);
    double* Gr  = (double*)malloc(sizeof(double) * d * d);   /* the chunk's gradient */
    double* e   = (double*)malloc(sizeof(double) * d);
    memcpy(W, W0, sizeof(double) * d * d);
    if (M0) memcpy(Mom, M0, sizeof(double) * d * d);
    else memset(Mom, 0, sizeof(double) * d * d);

    for (int c0 = 0; c0 < T; c0 += chunk) {
        int c1 = c0 + chunk < T ? c0 + chunk : T;
        memset(Gr, 0, sizeof(double) * d * d);
        for (int t = c0; t < c1; ++t) {
            const double* k = K + (size_t)t * d;
            const double* q = Q + (size_t)t * d;
            const double* v = V + (size_t)t * d;
            const double et = eta ? eta[t] : eta_scalar;
            double* z = Z + (size_t)t * d;
            for (int i = 0; i < d; ++i) {
                double se = 0.0, sz = 0.0;
                for (int j = 0; j < d; ++j) {
                    se += W[i * d + j] * k[j];
                    sz += W[i * d + j] * q[j];
                }
                e[i] = se - v[i];
                z[i] = sz;
            }
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) Gr[i * d + j] += et * e[i] * k[j];
        }
        for (int i = 0; i < d * d; ++i) {
            Mom[i] = beta * Mom[i] + (1.0 - beta) * Gr[i];
            W[i] -= Mom[i];
        }
    }
    memcpy(W_out, W, sizeof(double) * d * d);
    memcpy(M_out, Mom, sizeof(double) * d * d);
    free(W); free(Mom); free(Gr); free(e);
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear with a bias, and optionally LayerNorm and a residual inside f,  */
/* one slice.  diosapp "Test-Time Training (TTT) guide" §3 gives the inner    */
/* linear model as f(x) = W x + b; the 125M ablation of PaperTrace "5 ·      */
/* TestingTime 训练与长上下文" §3.1 adds LN                                   */
/* and a residual inside f, read here as f(x) = x + LN(W x + b) with          */
/* LN(u) = g * (u - mean(u)) / sqrt(var(u) + eps) + beta over the d features  */
/* (g, beta fixed: they belong to the outer model).  W and b are the state:  */
/* per token, at the chunk-start (Wc, bc),                                   */
/*   u = Wc k + bc,  r = f(k) - v,  grad_u = dl/du (through LN when present), */
/*   G += eta grad_u k^T,  gb += eta grad_u,  z = f_{Wc - G, bc - gb}(q),      */
/* and at the chunk end W = Wc - G, b = bc - gb.  lnw == NULL: f(x) = W x + b. */
/* ------------------------------------------------------------------------ */
/* LN of u over d features: writes the normalised uhat and returns 1/sigma.  */
static double ln_normalise(const double* u, double* uhat, int d, double eps)
{
    double mu = 0.0, var = 0.0;
    for (int i = 0; i < d; ++i) mu += u[i];
    mu /= d;
    for (int i = 0; i < d; ++i) var += (u[i] - mu) * (u[i] - mu);
    var /= d;
    const double rs = 1.0 / sqrt(var + eps);
    for (int i = 0; i < d; ++i) uhat[i] = (u[i] - mu) * rs;
    return rs;
}

static void linear_ln_slice(const double* K, const double* Q, const double* V,
                            const double* eta, double eta_scalar,
                            const double* W0, const double* b0,
                            const double* lnw, const double* lnb, double eps,
                            double* Z, double* W_out, double* b_out, int T, int d, int chunk)
{
    double* W  = (double*)malloc(sizeof(double) * d * d);
    double* Wc = (double*)malloc(sizeof(double) * d * d);
    double* G  = (double*)malloc(sizeof(double) * d * d);
    double* b  = (double*)malloc(sizeof(double) * d);
    double* bc = (double*)malloc(sizeof(double) * d);
    double* gb = (double*)malloc(sizeof(double) * d);
    double* u  = (double*)malloc(sizeof(double) * d);
    double* uh = (double*)malloc(sizeof(double) * d);
    double* gu = (double*)malloc(sizeof(double) * d);
    memcpy(W, W0, sizeof(double) * d * d);
    memcpy(b, b0, sizeof(double) * d);

    for (int c0 = 0; c0 < T; c0 += chunk) {
        int c1 = c0 + chunk < T ? c0 + chunk : T;
        memcpy(Wc, W, sizeof(double) * d * d);
        memcpy(bc, b, sizeof(double) * d);
        memset(G, 0, sizeof(double) * d * d);
        memset(gb, 0, sizeof(double) * d);
        for (int t = c0; t < c1; ++t) {
            const double* k = K + (size_t)t * d;
            const double* q = Q + (size_t)t * d;
            const double* v = V + (size_t)t * d;
            const double et = eta ? eta[t] : eta_scalar;
            /* pre-activation at the chunk-start state */
            for (int i = 0; i < d; ++i) {
                double acc = bc[i];
                for (int j = 0; j < d; ++j) acc += Wc[i * d + j] * k[j];
                u[i] = acc;
            }
            if (lnw) {
                /* r = k + LN(u) - v; dl/duhat = g * r; back through the normalisation:
                 * dl/du = (1/sigma) (h - mean(h) - uhat mean(h uhat)), h = dl/duhat */
                const double rs = ln_normalise(u, uh, d, eps);
                double mh = 0.0, mhu = 0.0;
                for (int i = 0; i < d; ++i) {
                    const double r = k[i] + lnw[i] * uh[i] + lnb[i] - v[i];
                    gu[i] = lnw[i] * r;
                    mh += gu[i];
                    mhu += gu[i] * uh[i];
                }
                mh /= d;
                mhu /= d;
                for (int i = 0; i < d; ++i) gu[i] = rs * (gu[i] - mh - uh[i] * mhu);
            } else {
                for (int i = 0; i < d; ++i) gu[i] = u[i] - v[i];
            }
            for (int i = 0; i < d; ++i) {
                for (int j = 0; j < d; ++j) G[i * d + j] += et * gu[i] * k[j];
                gb[i] += et * gu[i];
            }
            /* read with the chunk's updates up to and including this token */
            for (int i = 0; i < d; ++i) {
                double acc = bc[i] - gb[i];
                for (int j = 0; j < d; ++j) acc += (Wc[i * d + j] - G[i * d + j]) * q[j];
                u[i] = acc;
            }
            double* z = Z + (size_t)t * d;
            if (lnw) {
                ln_normalise(u, uh, d, eps);
                for (int i = 0; i < d; ++i) z[i] = q[i] + lnw[i] * uh[i] + lnb[i];
            } else {
                for (int i = 0; i < d; ++i) z[i] = u[i];
            }
        }
        for (int i = 0; i < d * d; ++i) W[i] = Wc[i] - G[i];
        for (int i = 0; i < d; ++i) b[i] = bc[i] - gb[i];
    }
    memcpy(W_out, W, sizeof(double) * d * d);
    memcpy(b_out, b, sizeof(double) * d);
    free(W); free(Wc); free(G); free(b); free(bc); free(gb); free(u); free(uh); free(gu);
}

/* ------------------------------------------------------------------------ */
/* Vector-Jacobian product of the TTT-Linear scan, one slice: the gradient of */
/* L = <dZ, Z> + <dW_T, W_T> with respect to K, Q, V, every token's eta and W0. */
/* Reverse mode through the same per-token loop as linear_slice (PaperTrace   */
/* "5 · TestingTime 训练与长上下文" §1.1, §2.1, §2.3), one chunk at a time from */
/* the last: with Wc the chunk-start state, G_t the chunk's accumulated update */
/* after token t, and adjoints written dX,                                    */
/*   W_next = Wc - G_last       : dWc = dW_next,  dG = -dW_next               */
/*   z_t = (Wc - G_t) q_t       : dWc += dz q^T,  dG -= dz q^T,               */
/*                                dq = (Wc - G_t)^T dz                         */
/*   G_t = G_{t-1} + eta e k^T  : deta = e^T dG k, de = eta dG k,             */
/*                                dk = eta dG^T e  (dG flows on to G_{t-1})    */
/*   e_t = Wc k_t - v_t         : dWc += de k^T,  dk += Wc^T de,  dv = -de     */
/* and dW_next of the previous chunk is this chunk's dWc.  The chunk-start    */
/* states come from a forward pass kept whole; G_{t-1} is G_t minus token t's  */
/* term.  deta_t is the gradient for token t's eta also when one scalar eta   */
/* serves every token (the scalar's gradient is then the sum over tokens).    */
/* ------------------------------------------------------------------------ */
static void linear_bwd_slice(const double* K, const double* Q, const double* V,
                             const double* eta, double eta_scalar, const double* W0,
                             const double* dZ, const double* dWT,
                             double* dK, double* dQ, double* dV, double* deta, double* dW0,
                             int T, int d, int chunk)
{
    const size_t dd = (size_t)d * d;
    const int nch = (T + chunk - 1) / chunk;
    double* Wst = (double*)malloc(sizeof(double) * dd * nch);  /* chunk-start states */
    double* W   = (double*)malloc(sizeof(double) * dd);
    double* G   = (double*)malloc(sizeof(double) * dd);
    double* dW  = (double*)malloc(sizeof(double) * dd);         /* adjoint of W_next  */
    double* dWc = (double*)malloc(sizeof(double) * dd);
    double* dG  = (double*)malloc(sizeof(double) * dd);
    double* E   = (double*)malloc(sizeof(double) * (size_t)chunk * d);
    double* de  = (double*)malloc(sizeof(double) * d);

    /* forward pass: the chunk-start states */
    memcpy(W, W0, sizeof(double) * dd);
    for (int c = 0; c < nch; ++c) {
        const int c0 = c * chunk, c1 = c0 + chunk < T ? c0 + chunk : T;
        double* Wc = Wst + (size_t)c * dd;
        memcpy(Wc, W, sizeof(double) * dd);
        memset(G, 0, sizeof(double) * dd);
        for (int t = c0; t < c1; ++t) {
            const double* k = K + (size_t)t * d;
            const double* v = V + (size_t)t * d;
            const double et = eta ? eta[t] : eta_scalar;
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += Wc[i * d + j] * k[j];
                const double ei = acc - v[i];
                for (int j = 0; j < d; ++j) G[i * d + j] += et * ei * k[j];
            }
        }
        for (size_t i = 0; i < dd; ++i) W[i] = Wc[i] - G[i];
    }

    /* reverse pass */
    if (dWT) memcpy(dW, dWT, sizeof(double) * dd);
    else memset(dW, 0, sizeof(double) * dd);
    for (int c = nch - 1; c >= 0; --c) {
        const int c0 = c * chunk, c1 = c0 + chunk < T ? c0 + chunk : T;
        const double* Wc = Wst + (size_t)c * dd;
        /* e_t for the chunk's tokens and the chunk's whole update G */
        memset(G, 0, sizeof(double) * dd);
        for (int t = c0; t < c1; ++t) {
            const double* k = K + (size_t)t * d;
            const double* v = V + (size_t)t * d;
            const double et = eta ? eta[t] : eta_scalar;
            double* e = E + (size_t)(t - c0) * d;
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += Wc[i * d + j] * k[j];
                e[i] = acc - v[i];
            }
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) G[i * d + j] += (et * e[i]) * k[j];
        }
        /* W_next = Wc - G */
        for (size_t i = 0; i < dd; ++i) {
            dWc[i] = dW[i];
            dG[i] = -dW[i];
        }
        for (int t = c1 - 1; t >= c0; --t) {
            const double* k = K + (size_t)t * d;
            const double* q = Q + (size_t)t * d;
            const double* dz = dZ + (size_t)t * d;
            const double et = eta ? eta[t] : eta_scalar;
            const double* e = E + (size_t)(t - c0) * d;
            double* dk = dK + (size_t)t * d;
            double* dq = dQ + (size_t)t * d;
            double* dv = dV + (size_t)t * d;
            /* z_t = (Wc - G_t) q_t */
            for (int j = 0; j < d; ++j) {
                double acc = 0.0;
                for (int i = 0; i < d; ++i) acc += (Wc[i * d + j] - G[i * d + j]) * dz[i];
                dq[j] = acc;
            }
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) {
                    dWc[i * d + j] += dz[i] * q[j];
                    dG[i * d + j] -= dz[i] * q[j];
                }
            /* G_t = G_{t-1} + eta_t e_t k_t^T */
            double sdeta = 0.0;
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += dG[i * d + j] * k[j];
                sdeta += e[i] * acc;
                de[i] = et * acc;
            }
            deta[t] = sdeta;
            for (int j = 0; j < d; ++j) {
                double acc = 0.0;
                for (int i = 0; i < d; ++i) acc += dG[i * d + j] * e[i];
                dk[j] = et * acc;
            }
            /* e_t = Wc k_t - v_t */
            for (int j = 0; j < d; ++j) {
                double acc = 0.0;
                for (int i = 0; i < d; ++i) acc += Wc[i * d + j] * de[i];
                dk[j] += acc;
            }
            for (int i = 0; i < d; ++i) {
                dv[i] = -de[i];
                for (int j = 0; j < d; ++j) dWc[i * d + j] += de[i] * k[j];
            }
            /* back to G_{t-1} */
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) G[i * d + j] -= et * e[i] * k[j];
        }
        memcpy(dW, dWc, sizeof(double) * dd);
    }
    memcpy(dW0, dW, sizeof(double) * dd);
    free(Wst); free(W); free(G); free(dW); free(dWc); free(dG); free(E); free(de);
}

/* ------------------------------------------------------------------------ */
/* GELU, exact erf form: gelu(x) = x * Phi(x), Phi the standard normal CDF.  */
/* diosapp "Test-Time Training (TTT) guide" §3 names GELU; the erf form is   */
/* the reading taken here.                                                   */
/* ------------------------------------------------------------------------ */
double ttt_oracle_gelu(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/* d/dx [x Phi(x)] = Phi(x) + x phi(x), phi the standard normal density. */
double ttt_oracle_gelu_prime(double x)
{
    const double inv_sqrt_2pi = 0.39894228040143267794;
    return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * inv_sqrt_2pi * exp(-0.5 * x * x);
}

/* ------------------------------------------------------------------------ */
/* TTT-MLP, one (batch, head) slice.                                         */
/* f(x) = W2 gelu(W1 x + b1) + b2, hidden width `hidden` (4d on the page,    */
/* diosapp guide §3).  Per token, explicit backprop of 1/2||f(k) - v||^2 at  */
/* the chunk-start parameters Ps:                                            */
/*   h = W1 k + b1, a = gelu(h), e = W2 a + b2 - v                           */
/*   dW2 = e a^T, db2 = e, delta = (W2^T e) * gelu'(h), dW1 = delta k^T,     */
/*   db1 = delta;   G += eta_t * grad;   z_t = f_{Ps - G}(q_t).              */
/* A NULL bias is absent: it stays zero and receives no update.             */
/* ------------------------------------------------------------------------ */
static void mlp_slice(const double* K, const double* Q, const double* V,
                      const double* eta, double eta_scalar,
                      const double* W1_0, const double* b1_0,
                      const double* W2_0, const double* b2_0,
                      double* Z, double* W1_o, double* b1_o,
                      double* W2_o, double* b2_o,
                      int T, int d, int hd, int chunk)
{
    size_t n1 = (size_t)hd * d, n2 = (size_t)d * hd;
    double* W1  = (double*)calloc(n1, sizeof(double));
    double* W2  = (double*)calloc(n2, sizeof(double));
    double* b1  = (double*)calloc(hd, sizeof(double));
    double* b2  = (double*)calloc(d, sizeof(double));
    double* W1s = (double*)calloc(n1, sizeof(double));
    double* W2s = (double*)calloc(n2, sizeof(double));
    double* b1s = (double*)calloc(hd, sizeof(double));
    double* b2s = (double*)calloc(d, sizeof(double));
    double* G1  = (double*)calloc(n1, sizeof(double));
    double* G2  = (double*)calloc(n2, sizeof(double));
    double* g1  = (double*)calloc(hd, sizeof(double));
    double* g2  = (double*)calloc(d, sizeof(double));
    double* h   = (double*)calloc(hd, sizeof(double));
    double* a   = (double*)calloc(hd, sizeof(double));
    double* dl  = (double*)calloc(hd, sizeof(double));
    double* e   = (double*)calloc(d, sizeof(double));
    double* hr  = (double*)calloc(hd, sizeof(double));

    memcpy(W1, W1_0, sizeof(double) * n1);
    memcpy(W2, W2_0, sizeof(double) * n2);
    if (b1_0) memcpy(b1, b1_0, sizeof(double) * hd);
    if (b2_0) memcpy(b2, b2_0, sizeof(double) * d);

    for (int c0 = 0; c0 < T; c0 += chunk) {
        int c1 = c0 + chunk < T ? c0 + chunk : T;
        memcpy(W1s, W1, sizeof(double) * n1);
        memcpy(W2s, W2, sizeof(double) * n2);
        memcpy(b1s, b1, sizeof(double) * hd);
        memcpy(b2s, b2, sizeof(double) * d);
        memset(G1, 0, sizeof(double) * n1);
        memset(G2, 0, sizeof(double) * n2);
        memset(g1, 0, sizeof(double) * hd);
        memset(g2, 0, sizeof(double) * d);
        for (int t = c0; t < c1; ++t) {
            const double* k = K + (size_t)t * d;
            const double* q = Q + (size_t)t * d;
            const double* v = V + (size_t)t * d;
            double et = eta ? eta[t] : eta_scalar;
            /* forward at the chunk-start parameters */
            for (int u = 0; u < hd; ++u) {
                double s = b1s[u];
                for (int j = 0; j < d; ++j) s += W1s[(size_t)u * d + j] * k[j];
                h[u] = s;
                a[u] = ttt_oracle_gelu(s);
            }
            for (int i = 0; i < d; ++i) {
                double s = b2s[i];
                for (int u = 0; u < hd; ++u) s += W2s[(size_t)i * hd + u] * a[u];
                e[i] = s - v[i];
            }
            /* backward */
            for (int u = 0; u < hd; ++u) {
                double s = 0.0;
                for (int i = 0; i < d; ++i) s += W2s[(size_t)i * hd + u] * e[i];
                dl[u] = s * ttt_oracle_gelu_prime(h[u]);
            }
            /* accumulate eta_t * gradient */
            for (int i = 0; i < d; ++i)
                for (int u = 0; u < hd; ++u) G2[(size_t)i * hd + u] += et * e[i] * a[u];
            for (int u = 0; u < hd; ++u)
                for (int j = 0; j < d; ++j) G1[(size_t)u * d + j] += et * dl[u] * k[j];
            if (b2_0) for (int i = 0; i < d; ++i) g2[i] += et * e[i];
            if (b1_0) for (int u = 0; u < hd; ++u) g1[u] += et * dl[u];
            /* read with the updated parameters Ps - G */
            for (int u = 0; u < hd; ++u) {
                double s = b1s[u] - g1[u];
                for (int j = 0; j < d; ++j)
                    s += (W1s[(size_t)u * d + j] - G1[(size_t)u * d + j]) * q[j];
                hr[u] = ttt_oracle_gelu(s);
            }
            double* z = Z + (size_t)t * d;
            for (int i = 0; i < d; ++i) {
                double s = b2s[i] - g2[i];
                for (int u = 0; u < hd; ++u)
                    s += (W2s[(size_t)i * hd + u] - G2[(size_t)i * hd + u]) * hr[u];
                z[i] = s;
            }
        }
        for (size_t i = 0; i < n1; ++i) W1[i] = W1s[i] - G1[i];
        for (size_t i = 0; i < n2; ++i) W2[i] = W2s[i] - G2[i];
        for (int u = 0; u < hd; ++u) b1[u] = b1s[u] - g1[u];
        for (int i = 0; i < d; ++i) b2[i] = b2s[i] - g2[i];
    }
    memcpy(W1_o, W1, sizeof(double) * n1);
    memcpy(W2_o, W2, sizeof(double) * n2);
    if (b1_o) memcpy(b1_o, b1, sizeof(double) * hd);
    if (b2_o) memcpy(b2_o, b2, sizeof(double) * d);

    free(W1); free(W2); free(b1); free(b2); free(W1s); free(W2s); free(b1s); free(b2s);
    free(G1); free(G2); free(g1); free(g2); free(h); free(a); free(dl); free(e); free(hr);
}

/* ------------------------------------------------------------------------ */
/* Thread pool over (batch, head) slices.                                    */
/* ------------------------------------------------------------------------ */
typedef struct {
    int is_mlp, is_bwd, read_start, is_ln, is_mom;
    const double *K, *Q, *V, *eta, *W0, *W1, *b1, *W2, *b2, *dZ, *dWT, *b0, *lnw, *lnb, *M0;
    double eta_scalar, eps, beta;
    double *Z, *W_out, *W1_o, *b1_o, *W2_o, *b2_o, *dK, *dQ, *dV, *deta, *dW0;
    int BH, T, d, hd, chunk, nthreads, tid;
} job_t;

static void* worker(void* arg)
{
    const job_t* j = (const job_t*)arg;
    size_t td = (size_t)j->T * j->d;
    for (int s = j->tid; s < j->BH; s += j->nthreads) {
        const double* eta = j->eta ? j->eta + (size_t)s * j->T : NULL;
        if (j->is_mom) {
            size_t dd = (size_t)j->d * j->d;
            linear_momentum_slice(j->K + s * td, j->Q + s * td, j->V + s * td, eta,
                                  j->eta_scalar, j->W0 + s * dd, j->M0 ? j->M0 + s * dd : NULL,
                                  j->beta, j->Z + s * td, j->W_out + s * dd, j->W1_o + s * dd,
                                  j->T, j->d, j->chunk);
        } else if (j->is_ln) {
            size_t dd = (size_t)j->d * j->d;
            linear_ln_slice(j->K + s * td, j->Q + s * td, j->V + s * td, eta, j->eta_scalar,
                            j->W0 + s * dd, j->b0 + (size_t)s * j->d,
                            j->lnw ? j->lnw + (size_t)s * j->d : NULL,
                            j->lnb ? j->lnb + (size_t)s * j->d : NULL, j->eps,
                            j->Z + s * td, j->W_out + s * dd, j->b1_o + (size_t)s * j->d,
                            j->T, j->d, j->chunk);
        } else if (j->is_bwd) {
            size_t dd = (size_t)j->d * j->d;
            linear_bwd_slice(j->K + s * td, j->Q + s * td, j->V + s * td, eta, j->eta_scalar,
                             j->W0 + s * dd, j->dZ + s * td, j->dWT ? j->dWT + s * dd : NULL,
                             j->dK + s * td, j->dQ + s * td, j->dV + s * td,
                             j->deta + (size_t)s * j->T, j->dW0 + s * dd,
                             j->T, j->d, j->chunk);
        } else if (!j->is_mlp) {
            size_t dd = (size_t)j->d * j->d;
            linear_slice(j->K + s * td, j->Q + s * td, j->V + s * td, eta, j->eta_scalar,
                         j->W0 + s * dd, j->Z + s * td, j->W_out + s * dd,
                         j->T, j->d, j->chunk, j->read_start);
        } else {
            size_t n1 = (size_t)j->hd * j->d;
            mlp_slice(j->K + s * td, j->Q + s * td, j->V + s * td, eta, j->eta_scalar,
                      j->W1 + s * n1, j->b1 ? j->b1 + (size_t)s * j->hd : NULL,
                      j->W2 + s * n1, j->b2 ? j->b2 + (size_t)s * j->d : NULL,
                      j->Z + s * td, j->W1_o + s * n1,
                      j->b1_o ? j->b1_o + (size_t)s * j->hd : NULL,
                      j->W2_o + s * n1,
                      j->b2_o ? j->b2_o + (size_t)s * j->d : NULL,
                      j->T, j->d, j->hd, j->chunk);
        }
    }
    return NULL;
}

static int run_pool(job_t* proto)
{
    int nt = proto->nthreads;
    if (nt <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nt = n > 0 ? (int)n : 1;
    }
    if (nt > proto->BH) nt = proto->BH;
    if (nt < 1) nt = 1;
    job_t* jobs = (job_t*)malloc(sizeof(job_t) * nt);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nt);
    for (int i = 0; i < nt; ++i) {
        jobs[i] = *proto;
        jobs[i].nthreads = nt;
        jobs[i].tid = i;
    }
    for (int i = 1; i < nt; ++i) pthread_create(&th[i], NULL, worker, &jobs[i]);
    worker(&jobs[0]);
    for (int i = 1; i < nt; ++i) pthread_join(th[i], NULL);
    free(jobs); free(th);
    return nt;
}

int ttt_oracle_linear(const double* K, const double* Q, const double* V,
                      const double* eta, double eta_scalar, const double* W0,
                      double* Z, double* W_out,
                      int BH, int T, int d, int chunk, int nthreads)
{
    return ttt_oracle_linear_read(K, Q, V, eta, eta_scalar, W0, Z, W_out, BH, T, d, chunk, 0,
                                  nthreads);
}

int ttt_oracle_linear_read(const double* K, const double* Q, const double* V,
                           const double* eta, double eta_scalar, const double* W0,
                           double* Z, double* W_out,
                           int BH, int T, int d, int chunk, int read_start, int nthreads)
{
    if (!K || !Q || !V || !W0 || !Z || !W_out) return -1;
    if (BH <= 0 || T <= 0 || d <= 0 || chunk <= 0) return -1;
    if (read_start != 0 && read_start != 1) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.read_start = read_start;
    j.K = K; j.Q = Q; j.V = V; j.eta = eta; j.eta_scalar = eta_scalar; j.W0 = W0;
    j.Z = Z; j.W_out = W_out; j.BH = BH; j.T = T; j.d = d; j.chunk = chunk;
    j.nthreads = nthreads;
    return run_pool(&j);
}

int ttt_oracle_linear_momentum(const double* K, const double* Q, const double* V,
                               const double* eta, double eta_scalar, const double* W0,
                               const double* M0, double beta,
                               double* Z, double* W_out, double* M_out,
                               int BH, int T, int d, int chunk, int nthreads)
{
    if (!K || !Q || !V || !W0 || !Z || !W_out || !M_out) return -1;
    if (BH <= 0 || T <= 0 || d <= 0 || chunk <= 0 || !(beta >= 0.0 && beta < 1.0)) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.is_mom = 1;
    j.K = K; j.Q = Q; j.V = V; j.eta = eta; j.eta_scalar = eta_scalar; j.W0 = W0;
    j.M0 = M0; j.beta = beta;
    j.Z = Z; j.W_out = W_out; j.W1_o = M_out;
    j.BH = BH; j.T = T; j.d = d; j.chunk = chunk;
    j.nthreads = nthreads;
    return run_pool(&j);
}

int ttt_oracle_linear_ln(const double* K, const double* Q, const double* V,
                         const double* eta, double eta_scalar,
                         const double* W0, const double* b0,
                         const double* ln_weight, const double* ln_bias, double eps,
                         double* Z, double* W_out, double* b_out,
                         int BH, int T, int d, int chunk, int nthreads)
{
    if (!K || !Q || !V || !W0 || !b0 || !Z || !W_out || !b_out) return -1;
    if ((ln_weight == NULL) != (ln_bias == NULL)) return -1;
    if (BH <= 0 || T <= 0 || d <= 0 || chunk <= 0 || !(eps > 0.0)) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.is_ln = 1;
    j.K = K; j.Q = Q; j.V = V; j.eta = eta; j.eta_scalar = eta_scalar; j.W0 = W0; j.b0 = b0;
    j.lnw = ln_weight; j.lnb = ln_bias; j.eps = eps;
    j.Z = Z; j.W_out = W_out; j.b1_o = b_out;
    j.BH = BH; j.T = T; j.d = d; j.chunk = chunk;
    j.nthreads = nthreads;
    return run_pool(&j);
}

int ttt_oracle_linear_bwd(const double* K, const double* Q, const double* V,
                          const double* eta, double eta_scalar, const double* W0,
                          const double* dZ, const double* dW_T,
                          double* dK, double* dQ, double* dV, double* deta, double* dW0,
                          int BH, int T, int d, int chunk, int nthreads)
{
    if (!K || !Q || !V || !W0 || !dZ || !dK || !dQ || !dV || !deta || !dW0) return -1;
    if (BH <= 0 || T <= 0 || d <= 0 || chunk <= 0) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.is_bwd = 1;
    j.K = K; j.Q = Q; j.V = V; j.eta = eta; j.eta_scalar = eta_scalar; j.W0 = W0;
    j.dZ = dZ; j.dWT = dW_T; j.dK = dK; j.dQ = dQ; j.dV = dV; j.deta = deta; j.dW0 = dW0;
    j.BH = BH; j.T = T; j.d = d; j.chunk = chunk;
    j.nthreads = nthreads;
    return run_pool(&j);
}

int ttt_oracle_mlp(const double* K, const double* Q, const double* V,
                   const double* eta, double eta_scalar,
                   const double* W1, const double* b1,
                   const double* W2, const double* b2,
                   double* Z, double* W1_out, double* b1_out,
                   double* W2_out, double* b2_out,
                   int BH, int T, int d, int hidden, int chunk, int nthreads)
{
    if (!K || !Q || !V || !W1 || !W2 || !Z || !W1_out || !W2_out) return -1;
    if ((b1 == NULL) != (b1_out == NULL) || (b2 == NULL) != (b2_out == NULL)) return -1;
    if (BH <= 0 || T <= 0 || d <= 0 || hidden <= 0 || chunk <= 0) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.is_mlp = 1;
    j.K = K; j.Q = Q; j.V = V; j.eta = eta; j.eta_scalar = eta_scalar;
    j.W1 = W1; j.b1 = b1; j.W2 = W2; j.b2 = b2;
    j.Z = Z; j.W1_o = W1_out; j.b1_o = b1_out; j.W2_o = W2_out; j.b2_o = b2_out;
    j.BH = BH; j.T = T; j.d = d; j.hd = hidden; j.chunk = chunk;
    j.nthreads = nthreads;
    return run_pool(&j);
}
