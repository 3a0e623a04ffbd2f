// TTT-MLP forward scan on gfx950 matrix cores: d = 64, hidden 256, chunks of at
// most 16 tokens, bf16 I/O, fp16 matrix-core operands, fp32 state.
//
// Model and update: f(x) = W2 gelu(W1 x + b1) + b2 (diosapp "Test-Time Training
// (TTT) guide" §3: two layers, 4x hidden, GELU), loss 1/2||f(k) - v||^2, every
// gradient of a chunk at the chunk-start parameters, token t reads with the
// chunk's updates up to and including its own (PaperTrace "5 · TestingTime 训练与
// 长上下文" §1.1, §2.3).  Dual form of one chunk (u hidden, o/i features, s/t
// tokens, U[s,t] = [s <= t]):
//   H  = W1 K + b1,  A = gelu(H),  E = W2 A + b2 - V,  D = (W2^T E) * gelu'(H)
//   H' = W1 Q + b1 - D diag(eta) (U * (K^T Q + 1)),   A' = gelu(H')
//   Z  = W2 A' + b2 - E diag(eta) (U * (A^T A' + 1))
//   W1 -= D diag(eta) K^T,  b1 -= D eta,  W2 -= E diag(eta) A^T,  b2 -= E eta
// (the +1 terms are those of the biases and vanish for a model without them).
//
// Operands are fp16 (inputs converted exactly from bf16, state and gradients
// rounded to nearest): the state takes about 500 updates per sequence at the
// reference sizes and bf16's 8-bit significand let their rounding errors
// accumulate to ~2% of the state; fp16's 11 bits keep it ~8x smaller at the
// same matrix-core rate.  The fp16 operands are K, Q, W1, W2, A and A', E, the
// token scores and the eta-scaled gradients (-eta E and -eta D: D itself, a sum of
// |W2| |E| over the output features, can pass fp16's range where eta D does not);
// each must stay below 65504 in magnitude, or the outputs turn non-finite.
//
// One workgroup of four waves per (batch, head); wave w owns hidden units
// 64w .. 64w+63, i.e. rows of W1 and columns of W2.  Each product keeps one
// index in the lanes and the contracted one in the register slots (see
// mfma_common.h).  W2 is contracted over the hidden units for E and Z but over
// the output features for D: the fp32 state keeps it with the output feature in
// the lanes, and D takes the LDS transpose of its fp16 tiles each chunk.  Sums
// over all 256 hidden units (E, A^T A', W2 A') are formed as per-wave partials
// and added through LDS behind one barrier per chunk (the next chunk's H and E are
// read beside this chunk's Z, see the main loop).  A, A' and E change orientation
// through the LDS transpose read as well.  The next chunk's inputs are loaded
// while the current one is processed.
//
// GELU: gelu(x) = x Phi(x), gelu'(x) = Phi(x) + x phi(x), with erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26
// (|error| <= 1.5e-7), using the hardware exp2 and reciprocal.
#include <stdint.h>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kH = 256;
constexpr int kWaves = 4;
constexpr int kUB = 4;          // 16-unit hidden blocks per wave
constexpr int kNB = kD / 16;    // 16-feature blocks of d (input i and output o)

__device__ __forceinline__ float phi_erf(float x, float& e)
{
    // Phi(x) = 1/2 (1 + erf(x / sqrt 2)); e = exp(-x^2 / 2)
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    p *= t;
    e = __builtin_amdgcn_exp2f(-(z * z) * 1.44269504088896341f);
    const float erf_abs = fmaf(-p, e, 1.0f);
    return 0.5f + copysignf(0.5f * erf_abs, x);
}

__device__ __forceinline__ void gelu_pair(f32x4 h, f32x4& g, f32x4& gp)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float e;
        const float P = phi_erf(h[r], e);
        g[r] = h[r] * P;
        gp[r] = fmaf(h[r] * 0.39894228040143268f, e, P);
    }
}

__device__ __forceinline__ f32x4 gelu4(f32x4 h)
{
    f32x4 g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float e;
        g[r] = h[r] * phi_erf(h[r], e);
    }
    return g;
}

__device__ __forceinline__ f32x4 bf16x4_to_f32(u32x2 v)
{
    return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                 __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}

// shared LDS layout (bytes): per-wave private areas, then the partial sums
struct Lds {
    // private, per wave
    u32x2 tA[kWaves][kUB * 64];     // A (fp16) for the transpose
    u32x2 tA2[kWaves][kUB * 64];    // A'
    u32x2 tE[kWaves][kNB * 64];     // -eta E
    u32x2 tK[kWaves][kNB * 64];     // K tile for the W1 update operand
    u32x2 tW2[kWaves][kUB * kNB * 64];  // fp16 W2 tiles for the transpose to (u, o)
    float b2d[kWaves][kD];          // b2 update staging
    // shared partial sums (fp32, C/D layout, one f32x4 per lane), double-buffered
    // by chunk parity: a wave may write chunk c+1's partials while another still
    // reads chunk c's
    f32x4 Ep[2][kWaves][kNB][64];   // W2 A_{c+1}  (+ b2 - V_{c+1} from wave 0)
    f32x4 S3p[2][kWaves][64];       // A_c^T A_{c+1}
    f32x4 Zp[2][kWaves][kNB][64];   // W2 A'_c     (+ b2 from wave 0)
    f32x4 S2p[2][kWaves][64];       // A_c^T A'_c
};

// One chunk's inputs as loaded (bf16), one chunk ahead of their use.
struct ChunkIn {
    u32x4 k[kNB / 2], q[kNB / 2];   // K, Q rows (lane = token), pieces at 32m + 8g
    u32x2 v[kNB];                   // V[token][16ob + 4g ..], loaded by wave 0 only
    f32x4 er;                       // eta of tokens 4g + r
    float ec;                       // eta of token c
};

template <bool FULL, bool ETA_TOKEN, bool HAS_B1, bool HAS_B2>
__global__ __launch_bounds__(256) void mlp_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W1_0, const float* b1_0, const float* W2_0, const float* b2_0,
    uint16_t* __restrict__ Z, float* W1_out, float* b1_out, float* W2_out, float* b2_out,
    int T, int chunk)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    Lds& L = *reinterpret_cast<Lds*>(lds_raw);

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    const int slice = blockIdx.x;
    const size_t tok0 = (size_t)slice * T;
    const float* W1s = W1_0 + (size_t)slice * kH * kD;
    const float* W2s = W2_0 + (size_t)slice * kD * kH;
    const int ubase = 64 * w;   // first hidden unit of this wave

    // ---- state in C/D tiles ----
    // W1t[ub][ib]: lane (u, g), value r = W1[u][pi(ib, 4g + r)], u = ubase + 16ub + c
    // W2o[ob][ub]: lane (o, g), value r = W2[o][ubase + 16ub + 4g + r], o = 16ob + c
    // (W2 with the hidden unit in the lanes, needed for D, is the LDS transpose of
    // W2o's fp16 tiles, formed per chunk)
    f32x4 W1t[kUB][kNB], W2o[kNB][kUB];
    f32x4 b1r;      // b1[ubase + 16ub + c] for ub = 0..3
    f32x4 b2r[kNB]; // b2[16ob + 4g + r]
#pragma unroll
    for (int ub = 0; ub < kUB; ++ub) {
        const float* row = W1s + (size_t)(ubase + 16 * ub + c) * kD;
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) {
            W1t[ub][2 * m] = *(const f32x4*)(row + 32 * m + 8 * g);
            W1t[ub][2 * m + 1] = *(const f32x4*)(row + 32 * m + 8 * g + 4);
        }
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob)
            W2o[ob][ub] = *(const f32x4*)(W2s + (size_t)(16 * ob + c) * kH + ubase + 16 * ub + 4 * g);
        b1r[ub] = HAS_B1 ? b1_0[(size_t)slice * kH + ubase + 16 * ub + c] : 0.f;
    }
#pragma unroll
    for (int ob = 0; ob < kNB; ++ob)
        b2r[ob] = HAS_B2 ? *(const f32x4*)(b2_0 + (size_t)slice * kD + 16 * ob + 4 * g)
                         : f32x4{0, 0, 0, 0};

    const int step = chunk;   // <= 16
    const int nchunks = (T + step - 1) / step;
    // Loads one chunk's inputs; chunks past the end re-read the last one (their
    // values are never used).  Rows past a short chunk's end re-read row 0 of it;
    // their tokens are neutralised with eta = 0 where the chunk is used.
    auto load_in = [&](ChunkIn& t, int ci) {
        const int cc = ci < nchunks ? ci : nchunks - 1;
        const int s0 = cc * step;
        const int n = FULL ? 16 : min(step, T - s0);
        const size_t row = (tok0 + s0 + ((FULL || c < n) ? c : 0)) * kD;
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) {
            t.k[m] = *(const u32x4*)(K + row + 32 * m + 8 * g);
            t.q[m] = *(const u32x4*)(Q + row + 32 * m + 8 * g);
        }
        if (w == 0) {
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob) t.v[ob] = *(const u32x2*)(V + row + 16 * ob + 4 * g);
        } else {
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob) t.v[ob] = u32x2{0u, 0u};
        }
        if (ETA_TOKEN) {
            const float* e = eta + tok0 + s0;
#pragma unroll
            for (int r = 0; r < 4; ++r) t.er[r] = e[(FULL || 4 * g + r < n) ? 4 * g + r : 0];
            t.ec = e[(FULL || c < n) ? c : 0];
        } else {
            t.er = f32x4{eta_scalar, eta_scalar, eta_scalar, eta_scalar};
            t.ec = eta_scalar;
        }
    };
    auto to_f16 = [&](const u32x4 (&x)[kNB / 2], u32x4 (&y)[kNB / 2]) {
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) y[m] = bf16x8_to_f16x8(x[m]);
    };
    // fp16 state operands: W1 rows (B operand over the input features) and W2o tiles
    u32x4 W1f[kUB][kNB / 2];
    u32x2 W2f[kNB][kUB];
    auto pack_state = [&]() {
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub)
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m)
                W1f[ub][m] = pack_f16x8(W1t[ub][2 * m], W1t[ub][2 * m + 1]);
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob)
#pragma unroll
            for (int ub = 0; ub < kUB; ++ub) W2f[ob][ub] = pack_f16x4(W2o[ob][ub]);
    };
    auto w2pair = [&](int ob, int m) {
        return u32x4{W2f[ob][2 * m].x, W2f[ob][2 * m].y, W2f[ob][2 * m + 1].x, W2f[ob][2 * m + 1].y};
    };
    // A (fp16, lane = hidden unit) -> tokens in the lanes, hidden units in the slots
    auto transpose_a = [&](u32x2* buf, const u32x2 (&ab)[kUB], u32x4 (&ta)[kUB / 2]) {
        u32x2 t[kUB];
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) t[ub] = lds_transpose16(buf + ub * 64, ab[ub], lane);
#pragma unroll
        for (int m = 0; m < kUB / 2; ++m) ta[m] = u32x4{t[2 * m].x, t[2 * m].y, t[2 * m + 1].x, t[2 * m + 1].y};
    };
    // partial of W2 X (o x t) over this wave's units, plus `base` on wave 0
    auto w2_partial = [&](const u32x4 (&tx)[kUB / 2], int ob, f32x4 base) {
        f32x4 e = (w == 0) ? base : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < kUB / 2; ++m) e = mfma32h(w2pair(ob, m), tx[m], e);
        return e;
    };

    // ---- chunk 0's forward at the initial state: H, A, gelu'(H), E ----
    ChunkIn cur, nx, nx2;
    load_in(cur, 0);
    load_in(nx, 1);
    pack_state();
    u32x4 Kc[kNB / 2];          // K of the current chunk (fp16, lane = token)
    to_f16(cur.k, Kc);
    f32x4 G[kUB];               // gelu'(H_c)
    u32x2 Ab[kUB];              // A_c (fp16, lane = hidden unit, rows = tokens)
    u32x4 tAf[kUB / 2];         // A_c with tokens in the lanes
    f32x4 E[kNB];               // E_c (lanes = tokens, rows = output features)
    {
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) {
            f32x4 h = {b1r[ub], b1r[ub], b1r[ub], b1r[ub]};
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m) h = mfma32h(Kc[m], W1f[ub][m], h);
            f32x4 a;
            gelu_pair(h, a, G[ub]);
            Ab[ub] = pack_f16x4(a);
        }
        transpose_a(L.tA[w], Ab, tAf);
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob)
            L.Ep[1][w][ob][lane] = w2_partial(tAf, ob, b2r[ob] - bf16x4_to_f32(cur.v[ob]));
        __syncthreads();
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob) {
            f32x4 e = L.Ep[1][0][ob][lane];
#pragma unroll
            for (int v = 1; v < kWaves; ++v) e += L.Ep[1][v][ob][lane];
            E[ob] = e;
        }
    }

    // Chunk c, from its start state and its forward (H_c, A_c, E_c): the backward
    // D_c, then two reads of the chunk's updated model -- Q_c (the output, causal
    // and inclusive) and K_{c+1} (the next chunk's forward; every token of chunk c
    // precedes it) -- and one barrier for all the sums over hidden units:
    //   H'      = W1 Q_c     + b1 - D_c diag(eta) (U * (K_c^T Q_c + 1))
    //   H_{c+1} = W1 K_{c+1} + b1 - D_c diag(eta) (K_c^T K_{c+1} + 1)
    //   Z_c     = W2 A'      + b2 - E_c diag(eta) (U * (A_c^T A' + 1))
    //   E_{c+1} = W2 A_{c+1} + b2 - V_{c+1} - E_c diag(eta) (A_c^T A_{c+1} + 1)
    // The state update itself is off the chain: only the next chunk's operands
    // need it.
    for (int ci = 0; ci < nchunks; ++ci) {
        const int s0 = ci * step;
        const int n = FULL ? 16 : min(step, T - s0);
        const int pb = ci & 1;
        load_in(nx2, ci + 2);
        u32x4 Qf[kNB / 2], Kn[kNB / 2];
        to_f16(cur.q, Qf);
        to_f16(nx.k, Kn);
        f32x4 er = cur.er;   // zero for padding tokens
        float ec = cur.ec;
        if (!FULL) {
#pragma unroll
            for (int r = 0; r < 4; ++r) er[r] = (4 * g + r < n) ? er[r] : 0.f;
            ec = (c < n) ? ec : 0.f;
        }

        // -eta E_c with o in the lanes and tokens in the slots
        u32x2 tE[kNB];
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob)
            tE[ob] = lds_transpose16(&L.tE[w][ob * 64], pack_f16x4(-ec * E[ob]), lane);
        // ---- D^T (t x u) = (E^T W2) * gelu'(H) ----
        u32x4 Ef[kNB / 2];
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) Ef[m] = pack_f16x8(E[2 * m], E[2 * m + 1]);
        u32x2 DSb[kUB];     // -eta D_c: the scaled gradient stays small where D may not
        f32x4 db1 = {0, 0, 0, 0};
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) {
            // W2 with lanes = hidden unit u, slots = output features (transpose read)
            u32x2 w2t[kNB];
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob)
                w2t[ob] = lds_transpose16(&L.tW2[w][(ub * kNB + ob) * 64], W2f[ob][ub], lane);
            f32x4 d = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m)
                d = mfma32h(Ef[m], u32x4{w2t[2 * m].x, w2t[2 * m].y, w2t[2 * m + 1].x,
                                         w2t[2 * m + 1].y}, d);
            d = d * G[ub];
            const f32x4 ds = -er * d;
            DSb[ub] = pack_f16x4(ds);
            if (HAS_B1) db1[ub] = ds[0] + ds[1] + ds[2] + ds[3];
        }
        // ---- scores of K_c against Q_c (causal) and K_{c+1} (all); -eta rides on D ----
        u32x2 S1q, S1k;
        {
            f32x4 sq = {0, 0, 0, 0}, sk = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m) {
                sq = mfma32h(Kc[m], Qf[m], sq);
                sk = mfma32h(Kc[m], Kn[m], sk);
            }
            f32x4 mq, mk;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mq[r] = (4 * g + r <= c) ? sq[r] + (HAS_B1 ? 1.f : 0.f) : 0.f;
                mk[r] = sk[r] + (HAS_B1 ? 1.f : 0.f);
            }
            S1q = pack_f16x4(mq);
            S1k = pack_f16x4(mk);
        }
        // ---- H' and H_{c+1}; A' = gelu(H'), A_{c+1} = gelu(H_{c+1}), G_{c+1} ----
        u32x2 A2b[kUB], An[kUB];
        f32x4 Gn[kUB];
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) {
            f32x4 hq = {b1r[ub], b1r[ub], b1r[ub], b1r[ub]};
            f32x4 hk = hq;
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m) {
                hq = mfma32h(Qf[m], W1f[ub][m], hq);
                hk = mfma32h(Kn[m], W1f[ub][m], hk);
            }
            hq = mfma16h(S1q, DSb[ub], hq);
            hk = mfma16h(S1k, DSb[ub], hk);
            A2b[ub] = pack_f16x4(gelu4(hq));
            f32x4 a;
            gelu_pair(hk, a, Gn[ub]);
            An[ub] = pack_f16x4(a);
        }
        u32x4 tA2f[kUB / 2], tAn[kUB / 2];
        transpose_a(L.tA2[w], A2b, tA2f);
        transpose_a(L.tA[w], An, tAn);
        // ---- per-wave partials of Z_c and E_{c+1} ----
        {
            f32x4 s2 = {0, 0, 0, 0}, s3 = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < kUB / 2; ++m) {
                s2 = mfma32h(tAf[m], tA2f[m], s2);
                s3 = mfma32h(tAf[m], tAn[m], s3);
            }
            L.S2p[pb][w][lane] = s2;
            L.S3p[pb][w][lane] = s3;
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob) {
                L.Zp[pb][w][ob][lane] = w2_partial(tA2f, ob, b2r[ob]);
                L.Ep[pb][w][ob][lane] = w2_partial(tAn, ob, b2r[ob] - bf16x4_to_f32(nx.v[ob]));
            }
        }
        __syncthreads();

        // ---- Z_c: wave w finishes output block w ----
        {
            f32x4 s2 = L.S2p[pb][0][lane];
#pragma unroll
            for (int v = 1; v < kWaves; ++v) s2 += L.S2p[pb][v][lane];
            f32x4 sm;
#pragma unroll
            for (int r = 0; r < 4; ++r) sm[r] = (4 * g + r <= c) ? s2[r] + (HAS_B2 ? 1.f : 0.f) : 0.f;
            f32x4 z = L.Zp[pb][0][w][lane];
#pragma unroll
            for (int v = 1; v < kWaves; ++v) z += L.Zp[pb][v][w][lane];
            z = mfma16h(tE[w], pack_f16x4(sm), z);
            if (FULL || c < n) *(u32x2*)(Z + (tok0 + s0 + c) * kD + 16 * w + 4 * g) = pack_bf16x4(z);
        }
        // ---- E_{c+1} (every wave, every output block) ----
        {
            f32x4 s3 = L.S3p[pb][0][lane];
#pragma unroll
            for (int v = 1; v < kWaves; ++v) s3 += L.S3p[pb][v][lane];
            const u32x2 s3b = pack_f16x4(s3 + (HAS_B2 ? 1.f : 0.f));
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob) {
                f32x4 e = L.Ep[pb][0][ob][lane];
#pragma unroll
                for (int v = 1; v < kWaves; ++v) e += L.Ep[pb][v][ob][lane];
                E[ob] = mfma16h(tE[ob], s3b, e);
            }
        }

        // ---- state updates (needed from the next chunk's operands on) ----
        {
            // K_c with input features in the lanes and tokens in the slots
            // (block ib holds K[token][pi(ib, 0..15)] row by row, 512 bytes)
            u32x2 Kt[kNB];
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m) {
                L.tK[w][(2 * m) * 64 + 4 * c + g] = lo_half(Kc[m]);
                L.tK[w][(2 * m + 1) * 64 + 4 * c + g] = hi_half(Kc[m]);
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int ib = 0; ib < kNB; ++ib) {
                auto p = (__attribute__((address_space(3))) s16x4*)(&L.tK[w][ib * 64] + lane);
                Kt[ib] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int ub = 0; ub < kUB; ++ub)
#pragma unroll
                for (int ib = 0; ib < kNB; ++ib) W1t[ub][ib] = mfma16h(Kt[ib], DSb[ub], W1t[ub][ib]);
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob)
#pragma unroll
                for (int ub = 0; ub < kUB; ++ub) W2o[ob][ub] = mfma16h(Ab[ub], tE[ob], W2o[ob][ub]);
            if (HAS_B1) {
#pragma unroll
                for (int ub = 0; ub < kUB; ++ub) {
                    float v = db1[ub];
                    v += __shfl_xor(v, 16);
                    v += __shfl_xor(v, 32);
                    b1r[ub] += v;
                }
            }
            if (HAS_B2) {
                // b2 -= sum_s eta_s E[o][s]: sum tE's four token slots and the four
                // lane groups, stage through LDS, read back in the rows-of-o layout
#pragma unroll
                for (int ob = 0; ob < kNB; ++ob) {
                    const f32x4 t = f16x4_to_f32(tE[ob]);
                    float v = t[0] + t[1] + t[2] + t[3];
                    v += __shfl_xor(v, 16);
                    v += __shfl_xor(v, 32);
                    if (g == 0) L.b2d[w][16 * ob + c] = v;
                }
                asm volatile("" ::: "memory");
#pragma unroll
                for (int ob = 0; ob < kNB; ++ob) b2r[ob] += *(const f32x4*)&L.b2d[w][16 * ob + 4 * g];
                asm volatile("" ::: "memory");
            }
        }
        pack_state();
        // ---- move to the next chunk ----
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) {
            G[ub] = Gn[ub];
            Ab[ub] = An[ub];
        }
#pragma unroll
        for (int m = 0; m < kUB / 2; ++m) tAf[m] = tAn[m];
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) Kc[m] = Kn[m];
        cur = nx;
        nx = nx2;
    }

    // ---- final state ----
    float* W1o = W1_out + (size_t)slice * kH * kD;
    float* W2o_ = W2_out + (size_t)slice * kD * kH;
#pragma unroll
    for (int ub = 0; ub < kUB; ++ub) {
        float* row = W1o + (size_t)(ubase + 16 * ub + c) * kD;
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) {
            *(f32x4*)(row + 32 * m + 8 * g) = W1t[ub][2 * m];
            *(f32x4*)(row + 32 * m + 8 * g + 4) = W1t[ub][2 * m + 1];
        }
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob)
            *(f32x4*)(W2o_ + (size_t)(16 * ob + c) * kH + ubase + 16 * ub + 4 * g) = W2o[ob][ub];
        if (HAS_B1 && g == 0) b1_out[(size_t)slice * kH + ubase + 16 * ub + c] = b1r[ub];
    }
    if (HAS_B2 && w == 0 && c == 0) {
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob)
            *(f32x4*)(b2_out + (size_t)slice * kD + 16 * ob + 4 * g) = b2r[ob];
    }
}

template <bool FULL, bool ETA_TOKEN, bool HAS_B1, bool HAS_B2>
hipError_t launch4(const MlpArgs& a, hipStream_t s)
{
    auto k = mlp_mfma_kernel<FULL, ETA_TOKEN, HAS_B1, HAS_B2>;
    const int lds = (int)sizeof(Lds);
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)a.BH), dim3(64 * kWaves), lds, s, (const uint16_t*)a.K,
                       (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta, a.eta_scalar, a.W1, a.b1,
                       a.W2, a.b2, (uint16_t*)a.Z, a.W1_out, a.b1_out, a.W2_out, a.b2_out, a.T,
                       a.chunk);
    return hipGetLastError();
}

template <bool FULL, bool ETA_TOKEN>
hipError_t launch_bias(const MlpArgs& a, hipStream_t s)
{
    if (a.b1 && a.b2) return launch4<FULL, ETA_TOKEN, true, true>(a, s);
    if (a.b1) return launch4<FULL, ETA_TOKEN, true, false>(a, s);
    if (a.b2) return launch4<FULL, ETA_TOKEN, false, true>(a, s);
    return launch4<FULL, ETA_TOKEN, false, false>(a, s);
}

}  // namespace

bool mlp_mfma_supported(int d, int chunk, int bf16)
{
    return bf16 && d == kD && chunk <= 16;
}

hipError_t launch_mlp_mfma(const MlpArgs& a, hipStream_t s)
{
    const bool full = a.chunk == 16 && a.T % 16 == 0;
    if (full) return a.eta ? launch_bias<true, true>(a, s) : launch_bias<true, false>(a, s);
    return a.eta ? launch_bias<false, true>(a, s) : launch_bias<false, false>(a, s);
}

}  // namespace ttt
