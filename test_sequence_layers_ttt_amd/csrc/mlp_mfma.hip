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
// One workgroup of eight waves per (batch, head), two per SIMD so that one
// wave's waits on the matrix cores and LDS are filled by the other's work; wave w
// owns hidden units 32w .. 32w+31, i.e. rows of W1 and columns of W2.  Each
// product keeps one index in the lanes and the contracted one in the register
// slots (see mfma_common.h).  W2 is contracted over the hidden units for E and Z
// but over the output features for D: the fp32 state keeps it with the output
// feature in the lanes, and D takes the LDS transpose of its fp16 tiles each
// chunk.  (Transposing on the matrix cores instead, as a product with the
// identity, measured 11% slower: it lengthens each wave's dependent chain.)
//
// Per chunk each wave forms its partials of Z_c and E_{c+1} over its own units,
// each with its share of the eta-weighted correction already added (the
// correction E diag(eta) (U * (A^T A' + 1)) is linear in the per-wave sums of
// A^T A'), and writes them to LDS.  After a barrier all 512 threads reduce the
// eight partials, two values each: the Z values go to memory with b2 added, the
// E values get b2 - V and are written back as the fp16 operands the next chunk
// reads (E and -eta E); the thread that owns an output feature also keeps that
// bias and adds the chunk's step, which wave 0 forms as -eta E times ones.  A second barrier publishes them.  K and Q of each chunk are staged once
// per workgroup in LDS as fp16 rows (two chunks ahead), and both the row operand
// and the transposed K come from that tile.
//
// GELU: gelu(x) = x Phi(x), gelu'(x) = Phi(x) + x phi(x).  Each workgroup first
// tabulates Phi and gelu' at 1024 points on [-8, 8) (step 1/64; erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26, |error| <=
// 1.5e-7, with the hardware exp2 and reciprocal) and then interpolates linearly:
// |error| <= 7.4e-6 in Phi and 2.4e-5 in gelu' (beyond +-8 the end values, where
// Phi is 0 or 1 to 6e-16).  That is far below the fp16 rounding of the
// activations, and it replaces a reciprocal, an exponential and about fifteen
// other operations per element by an LDS read and five operations.
#include <stdint.h>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int kD = 64;
constexpr int kH = 256;
constexpr int kWaves = 8;
constexpr int kUB = 2;          // 16-unit hidden blocks per wave
constexpr int kUW = 16 * kUB;   // hidden units per wave
constexpr int kNB = kD / 16;    // 16-feature blocks of d (input i and output o)
constexpr int kRing = 3;        // staged chunks: the current, the next, the one arriving
static_assert(kWaves * kUW == kH, "the waves cover the hidden units");

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

// Table of Phi and gelu' at x_i = -8 + i / 64: entry i holds (Phi(x_i),
// Phi(x_{i+1}) - Phi(x_i), gelu'(x_i), gelu'(x_{i+1}) - gelu'(x_i)).
constexpr int kTab = 1024;

__device__ __forceinline__ f32x4 gelu_tab_entry(int i)
{
    float e0, e1;
    const float x0 = -8.f + (float)i * (1.f / 64.f), x1 = x0 + 1.f / 64.f;
    const float p0 = phi_erf(x0, e0), p1 = phi_erf(x1, e1);
    const float g0 = fmaf(x0 * 0.39894228040143268f, e0, p0);
    const float g1 = fmaf(x1 * 0.39894228040143268f, e1, p1);
    return f32x4{p0, p1 - p0, g0, g1 - g0};
}

// table position of x: entry index (clamped to the table, 0 for a NaN) and the
// fraction of the step past it
__device__ __forceinline__ int gelu_tab_pos(float x, float& fr)
{
    // t in [0, 1023.999] (a NaN converts to 0), so the index needs no clamp
    const float t = __builtin_amdgcn_fmed3f(fmaf(x, 64.f, 512.f), 0.f, 1023.999f);
    fr = __builtin_amdgcn_fractf(t);
    return (int)t;
}

__device__ __forceinline__ void gelu_pair(const f32x4* tab, f32x4 h, f32x4& g, f32x4& gp)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float fr;
        const f32x4 e = tab[gelu_tab_pos(h[r], fr)];
        g[r] = h[r] * fmaf(e.y, fr, e.x);
        gp[r] = fmaf(e.w, fr, e.z);
    }
}

__device__ __forceinline__ f32x4 gelu4(const f32x4* tab, f32x4 h)
{
    f32x4 g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float fr;
        const f32x2 e = *reinterpret_cast<const f32x2*>(&tab[gelu_tab_pos(h[r], fr)]);
        g[r] = h[r] * fmaf(e.y, fr, e.x);
    }
    return g;
}

// LDS layout: staged inputs, per-wave transpose buffers, the shared fp16 E
// operands and the per-wave partial sums
struct Lds {
    f32x4 gtab[kTab];                   // Phi and gelu' for interpolation
    KQTile16<kD> kq[kRing];             // fp16 K and Q rows of three staged chunks
    float eta[kRing][16];               // their tokens' eta (0 past a short chunk's end)
    u32x2 tW2[kWaves][kUB * kNB * 64];  // per wave: fp16 W2 tiles for the transpose to (u, o)
    u32x2 tA[kWaves][kUB * 64];         // per wave: A (fp16) for the transpose
    u32x2 tA2[kWaves][kUB * 64];        // per wave: A'
    u32x2 tE[kNB * 64];                 // -eta E (fp16), the transpose read's source layout
    u32x4 Ef[2 * 64];                   // E (fp16) as the A operand of the D product
    float b2d[kD];                      // the chunk's b2 step, -sum_s eta_s E[o][s]
    f32x4 Ep[kWaves][kNB][64];          // per wave: W2 A_{c+1} - E diag(eta) (A_c^T A_{c+1} [+ 1])
    f32x4 Zp[kWaves][kNB][64];          // per wave: W2 A'_c  - E diag(eta) (U * (A_c^T A'_c [+ 1]))
};

template <bool FULL, bool ETA_TOKEN, bool HAS_B1, bool HAS_B2>
__global__ __launch_bounds__(64 * kWaves) void mlp_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W1_0, const float* b1_0, const float* W2_0, const float* b2_0,
    uint16_t* __restrict__ Z, float* W1_out, float* b1_out, float* W2_out, float* b2_out,
    int T, int chunk)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    Lds& L = *reinterpret_cast<Lds*>(lds_raw);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int slice = blockIdx.x;
    const size_t tok0 = (size_t)slice * T;
    const float* W1s = W1_0 + (size_t)slice * kH * kD;
    const float* W2s = W2_0 + (size_t)slice * kD * kH;
    const int ubase = kUW * w;   // first hidden unit of this wave
    const int step = chunk;      // <= 16
    const int nchunks = (T + step - 1) / step;

    // ---- state in C/D tiles ----
    // W1t[ub][ib]: lane (u, g), value r = W1[u][pi(ib, 4g + r)], u = ubase + 16ub + c,
    //              pi(2m + h, 4g + r) = 32m + 8g + 4h + r
    // W2o[ob][ub]: lane (o, g), value r = W2[o][ubase + 16ub + 4g + r], o = 16ob + c
    f32x4 W1t[kUB][kNB], W2o[kNB][kUB];
    float b1r[kUB];   // b1[ubase + 16ub + c]
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

    // ---- the reduction's share: two values of each 16 x 64 (token, output) tile ----
    // value pair p = tid of the C/D layout [ob][lane'][r]: ob = p / 128,
    // lane' = (p / 2) % 64, r = 2 (p % 2) + {0, 1}
    const int rv = 2 * tid;                    // first float of the pair in a partial
    const int rob = tid >> 7, rln = (tid >> 1) & 63, rrp = tid & 1;
    const int rtok = rln & 15;                 // token within the chunk
    const int rout = 16 * rob + 4 * (rln >> 4) + 2 * rrp;   // first output feature
    f32x2 b2v = {0.f, 0.f};
    if (HAS_B2) b2v = *(const f32x2*)(b2_0 + (size_t)slice * kD + rout);

    // ---- staging: thread t < 256 carries granule t % 128 of K (t < 128) or Q,
    // threads 256..271 the eta of one token ----
    const bool ld_kq = tid < 256;
    const int lwhich = (tid >> 7) & 1, lrow = (tid >> 3) & 15, lgr = tid & 7;
    const int lpos = lrow * (kD / 8) + (lgr ^ tile16_swizzle<kD>(lrow));
    const bool ld_eta = tid >= 256 && tid < 272;
    const int etok = tid - 256;
    auto chunk_n = [&](int cc) { return FULL ? 16 : min(step, T - cc * step); };
    auto stage_load = [&](int ci, u32x4& r, float& e) {
        const int cc = ci < nchunks ? ci : nchunks - 1;
        const int s0 = cc * step, n = chunk_n(cc);
        if (ld_kq) {
            const int row = (FULL || lrow < n) ? lrow : 0;
            r = *(const u32x4*)((lwhich ? Q : K) + (tok0 + s0 + row) * kD + 8 * lgr);
        }
        if (ld_eta) {
            if (ETA_TOKEN) e = (FULL || etok < n) ? eta[tok0 + s0 + etok] : 0.f;
            else e = (FULL || etok < n) ? eta_scalar : 0.f;
        }
    };
    auto stage_store = [&](int ci, const u32x4& r, float e) {
        const int sl = ci % kRing;
        if (ld_kq) L.kq[sl].g[lwhich][lpos] = bf16x8_to_f16x8(r);
        if (ld_eta) L.eta[sl][etok] = e;
    };
    // V of the reduction's pair for the chunk ci (clamped rows as above)
    auto v_load = [&](int ci) {
        const int cc = ci < nchunks ? ci : nchunks - 1;
        const int s0 = cc * step, n = chunk_n(cc);
        const int row = (FULL || rtok < n) ? rtok : 0;
        return *(const unsigned*)(V + (tok0 + s0 + row) * kD + rout);
    };

    // row operand of a staged tile: lane (c, g) gets granules 4m + g of row c
    auto row_operand = [&](const u32x4* t, u32x4 (&op)[kNB / 2]) {
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) op[m] = t[c * (kD / 8) + ((4 * m + g) ^ tile16_swizzle<kD>(c))];
    };
    // K with the input feature in the lanes and tokens 4g..4g+3 in the slots, for
    // the feature blocks ib of the W1t layout (transpose read of the staged rows)
    auto k_transposed = [&](const u32x4* t, u32x2 (&kt)[kNB]) {
        const int r = (lane >> 2) & 3, q = lane & 3;
        const int row = 4 * g + r;
        const u32x2* base = reinterpret_cast<const u32x2*>(t) + row * (2 * (kD / 8));
#pragma unroll
        for (int ib = 0; ib < kNB; ++ib) {
            auto pt = (__attribute__((address_space(3))) s16x4*)(
                base + 2 * ((4 * (ib >> 1) + q) ^ tile16_swizzle<kD>(row)) + (ib & 1));
            kt[ib] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(pt));
        }
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
    // A (fp16, lane = hidden unit) -> tokens in the lanes, hidden units in the slots
    auto transpose_a = [&](u32x2* buf, const u32x2 (&ab)[kUB], u32x4& ta) {
        u32x2 t[kUB];
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) t[ub] = lds_transpose16(buf + ub * 64, ab[ub], lane);
        ta = u32x4{t[0].x, t[0].y, t[1].x, t[1].y};
    };
    // W2 X (o x t) over this wave's 32 units
    auto w2_partial = [&](const u32x4& tx, int ob) {
        const u32x4 a = {W2f[ob][0].x, W2f[ob][0].y, W2f[ob][1].x, W2f[ob][1].y};
        return mfma32h(a, tx, f32x4{0, 0, 0, 0});
    };
    // the reduction of one partial set: this thread's pair, summed over the waves
    auto reduce_pair = [&](const f32x4 (*P)[kNB][64]) {
        const float* base = reinterpret_cast<const float*>(P) + rv;
        f32x2 s = *(const f32x2*)base;
#pragma unroll
        for (int v = 1; v < kWaves; ++v) s += *(const f32x2*)(base + v * (kNB * 64 * 4));
        return s;
    };
    // publish E (this thread's pair, token rtok of the chunk whose eta sits in
    // slot sl): as fp16 for the D product and, times -eta, for the transposes
    auto publish_e = [&](f32x2 e, int sl) {
        const float et = L.eta[sl][rtok];
        unsigned* ef = reinterpret_cast<unsigned*>(L.Ef);
        ef[((rob >> 1) * 64 + rln) * 4 + (rob & 1) * 2 + rrp] = pack_f16x2(e.x, e.y);
        unsigned* te = reinterpret_cast<unsigned*>(L.tE);
        te[(rob * 64 + 4 * rtok + (rln >> 4)) * 2 + rrp] = pack_f16x2(-et * e.x, -et * e.y);
    };

    // ---- prologue: the GELU table; stage chunks 0 and 1, hold chunk 2 ----
    for (int i = tid; i < kTab; i += 64 * kWaves) L.gtab[i] = gelu_tab_entry(i);
    u32x4 sr = {0u, 0u, 0u, 0u};
    float se = 0.f;
    stage_load(0, sr, se);
    stage_store(0, sr, se);
    stage_load(1, sr, se);
    stage_store(1, sr, se);
    stage_load(2, sr, se);
    unsigned vnext = v_load(0);
    pack_state();
    __syncthreads();

    // ---- chunk 0's forward at the initial state: H, A, gelu'(H), E ----
    f32x4 G[kUB];      // gelu'(H_c) of this wave's units
    u32x2 Ab[kUB];     // A_c (fp16, lane = hidden unit, rows = tokens)
    u32x4 tAf;         // A_c with tokens in the lanes
    {
        u32x4 Kc[kNB / 2];
        row_operand(L.kq[0].g[0], Kc);
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) {
            f32x4 h = {b1r[ub], b1r[ub], b1r[ub], b1r[ub]};
#pragma unroll
            for (int m = 0; m < kNB / 2; ++m) h = mfma32h(Kc[m], W1f[ub][m], h);
            f32x4 a;
            gelu_pair(L.gtab, h, a, G[ub]);
            Ab[ub] = pack_f16x4(a);
        }
        transpose_a(L.tA[w], Ab, tAf);
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob) L.Ep[w][ob][lane] = w2_partial(tAf, ob);
    }
    __syncthreads();
    {
        f32x2 e = reduce_pair(L.Ep);
        const unsigned v = vnext;
        e.x += b2v.x - __uint_as_float(v << 16);
        e.y += b2v.y - __uint_as_float(v & 0xffff0000u);
        publish_e(e, 0);
        vnext = v_load(1);
    }
    __syncthreads();

    // Chunk c, from its start state and its forward (H_c, A_c, E_c): the backward
    // D_c, then two reads of the chunk's updated model -- Q_c (the output, causal
    // and inclusive) and K_{c+1} (the next chunk's forward; every token of chunk c
    // precedes it):
    //   H'      = W1 Q_c     + b1 - D_c diag(eta) (U * (K_c^T Q_c + 1))
    //   H_{c+1} = W1 K_{c+1} + b1 - D_c diag(eta) (K_c^T K_{c+1} + 1)
    //   Z_c     = W2 A'      + b2 - E_c diag(eta) (U * (A_c^T A' + 1))
    //   E_{c+1} = W2 A_{c+1} + b2 - V_{c+1} - E_c diag(eta) (A_c^T A_{c+1} + 1)
    for (int ci = 0; ci < nchunks; ++ci) {
        const int s0 = ci * step;
        const int n = chunk_n(ci);
        const int sl = ci % kRing, sn = (ci + 1) % kRing;

        // the staged chunk ci + 2 goes to the slot chunk ci - 1 left (read before the
        // last barrier); chunk ci + 3 is fetched
        stage_store(ci + 2, sr, se);
        stage_load(ci + 3, sr, se);

        // E_c (fp16) and -eta E_c with o in the lanes and tokens in the slots
        u32x4 Ef[kNB / 2];
#pragma unroll
        for (int m = 0; m < kNB / 2; ++m) Ef[m] = L.Ef[m * 64 + lane];
        u32x2 tE[kNB];
#pragma unroll
        for (int ob = 0; ob < kNB; ++ob) {
            auto p = (__attribute__((address_space(3))) s16x4*)(&L.tE[ob * 64] + lane);
            tE[ob] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
        }
        const f32x4 er = *(const f32x4*)&L.eta[sl][4 * g];   // zero for padding tokens

        // ---- D^T (t x u) = (E^T W2) * gelu'(H), scaled by -eta ----
        u32x2 DSb[kUB];
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
            const f32x4 ds = -er * (d * G[ub]);
            DSb[ub] = pack_f16x4(ds);
        }
        // ---- scores of K_c against Q_c (causal) and K_{c+1} (all); -eta rides on D ----
        u32x4 Kc[kNB / 2], Qf[kNB / 2], Kn[kNB / 2];
        row_operand(L.kq[sl].g[0], Kc);
        row_operand(L.kq[sl].g[1], Qf);
        row_operand(L.kq[sn].g[0], Kn);
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
            A2b[ub] = pack_f16x4(gelu4(L.gtab, hq));
            f32x4 a;
            gelu_pair(L.gtab, hk, a, Gn[ub]);
            An[ub] = pack_f16x4(a);
        }
        u32x4 tA2f, tAn;
        transpose_a(L.tA2[w], A2b, tA2f);
        transpose_a(L.tA[w], An, tAn);
        // ---- this wave's partials of Z_c and E_{c+1}, corrections included (the
        // bias "+1" terms once, on wave 0) ----
        {
            const f32x4 s2 = mfma32h(tAf, tA2f, f32x4{0, 0, 0, 0});
            const f32x4 s3 = mfma32h(tAf, tAn, f32x4{0, 0, 0, 0});
            const float one = (HAS_B2 && w == 0) ? 1.f : 0.f;
            f32x4 sm;
#pragma unroll
            for (int r = 0; r < 4; ++r) sm[r] = (4 * g + r <= c) ? s2[r] + one : 0.f;
            const u32x2 smb = pack_f16x4(sm);
            const u32x2 s3b = pack_f16x4(s3 + one);
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob) {
                L.Zp[w][ob][lane] = mfma16h(tE[ob], smb, w2_partial(tA2f, ob));
                L.Ep[w][ob][lane] = mfma16h(tE[ob], s3b, w2_partial(tAn, ob));
            }
            if (HAS_B2 && w == 0) {
                // the b2 step: -eta E summed over the chunk's tokens, as a product
                // with ones (every token column of the result holds it)
                const u32x2 ones = {0x3C003C00u, 0x3C003C00u};
#pragma unroll
                for (int ob = 0; ob < kNB; ++ob) {
                    const f32x4 dl = mfma16h(tE[ob], ones, f32x4{0, 0, 0, 0});
                    if (c == 0) *(f32x4*)&L.b2d[16 * ob + 4 * g] = dl;
                }
            }
        }
        // ---- state updates (this wave's units; needed from the next chunk on) ----
        {
            u32x2 Kt[kNB];
            k_transposed(L.kq[sl].g[0], Kt);
#pragma unroll
            for (int ub = 0; ub < kUB; ++ub)
#pragma unroll
                for (int ib = 0; ib < kNB; ++ib) W1t[ub][ib] = mfma16h(Kt[ib], DSb[ub], W1t[ub][ib]);
#pragma unroll
            for (int ob = 0; ob < kNB; ++ob)
#pragma unroll
                for (int ub = 0; ub < kUB; ++ub) W2o[ob][ub] = mfma16h(Ab[ub], tE[ob], W2o[ob][ub]);
            if (HAS_B1) {
                // the b1 step, -eta D summed over the chunk's tokens: ones times
                // the same operand the W1 update takes (every row holds the sum)
                const u32x2 ones = {0x3C003C00u, 0x3C003C00u};
#pragma unroll
                for (int ub = 0; ub < kUB; ++ub)
                    b1r[ub] += mfma16h(ones, DSb[ub], f32x4{0, 0, 0, 0})[0];
            }
        }
        __syncthreads();

        // ---- reduction: Z_c to memory, E_{c+1} published, b2 stepped ----
        {
            f32x2 z = reduce_pair(L.Zp) + b2v;
            if (FULL || rtok < n) {
                unsigned* zp = reinterpret_cast<unsigned*>(Z + (tok0 + s0 + rtok) * kD + rout);
                *zp = pack_bf16x2(z.x, z.y);
            }
            f32x2 e = reduce_pair(L.Ep);
            const unsigned v = vnext;
            e.x += b2v.x - __uint_as_float(v << 16);
            e.y += b2v.y - __uint_as_float(v & 0xffff0000u);
            if (HAS_B2) b2v += *(const f32x2*)&L.b2d[rout];   // wave 0's sum over the tokens
            publish_e(e, sn);
            vnext = v_load(ci + 2);
        }
        pack_state();
#pragma unroll
        for (int ub = 0; ub < kUB; ++ub) {
            G[ub] = Gn[ub];
            Ab[ub] = An[ub];
        }
        tAf = tAn;
        __syncthreads();
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
    if (HAS_B2 && rtok == 0) *(f32x2*)(b2_out + (size_t)slice * kD + rout) = b2v;
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
