// TTT-Linear forward scan for large chunks (hundreds to thousands of tokens, the
// LaCT regime of PaperTrace "5 · TestingTime 训练与长上下文" §1.1 and §2.4), bf16
// I/O, fp32 state, d in {64, 128}.
//
// With E_c = W_c K_c - V_c (tokens as columns) the chunk update
//     W_{c+1} = W_c - E_c diag(eta) K_c^T = W_c - W_c P_c + B_c,
//     P_c = K_c diag(eta) K_c^T,   B_c = V_c diag(eta) K_c^T,
// is affine in W_c, and P_c, B_c (d x d) need no state.  Three kernels:
//   A  (parallel over every chunk): P_c and B_c on the matrix cores;
//   B  (one chain per (batch, head), split by 16 output rows): W_{c+1} from W_c,
//      storing every chunk-start state W_c;
//   C  (parallel over every chunk): the 16-token sub-tile dual form of the chunk
//      from its stored W_c, writing Z.
// Only the short d x d chain of kernel B is sequential; the long per-chunk work
// is spread over all chunks at once.
//
// Workspace, in this order: P (bf16, [BH*nchunks, d, d]), B (fp32, same shape),
// chunk-start states W_c (fp32, same shape).
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int kKStep = 32;   // tokens per contraction step of kernel A

// ---------------------------------------------------------------------------
// Kernel A.  One workgroup (d/16 waves) per (batch*head, chunk).  Per 32-token
// step the K and V rows are staged in LDS as row-major 16 x 16 bf16 blocks
// (block (token group, feature block)); the transpose read then yields operands
// with features in the lanes and tokens in the slots.
//   P tile:  D[i][j] = sum_s (eta K)[s][i] K[s][j]   -> lane j, rows i
//   B tile:  D[i][o] = sum_s K[s][i] (eta V)[s][o]   -> lane o, rows i
// Wave w owns input blocks i = 2 (w % (d/32)) + {0, 1} against output blocks
// j = (d/32) (w / (d/32)) + {0 .. d/32 - 1}: eight tiles of P and eight of B at
// d = 128, read through two A operands and d/16 B operands per step.  With a
// scalar eta, K itself is the A operand of both products (eta is applied at
// the end); per-token eta stages eta*K and eta*V as well.
// P is symmetric, so the tile's lane-j column is stored as row j of P; B's
// lane-o column is row o of B = V diag(eta) K^T.
// ---------------------------------------------------------------------------
template <int D, bool ETA_TOKEN>
__global__ __launch_bounds__(64 * (D / 16)) void bigchunk_gram_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar, uint16_t* __restrict__ Pout,
    float* __restrict__ Bout, int T, int chunk, int nchunks)
{
    constexpr int NB = D / 16;
    constexpr int NH = NB / 2;                  // output blocks per wave
    constexpr int BLK = 64;                     // u32x2 per 16 x 16 block
    constexpr int TILE = 2 * NB * BLK;          // u32x2 per 32-token tile
    constexpr int NT = ETA_TOKEN ? 3 : 2;       // staged tiles: K, (eta K,) V or eta V
    constexpr int TK = 0, TEK = ETA_TOKEN ? 1 : 0, TV = NT - 1;
    __shared__ u32x2 lds[2][NT][TILE];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int i0 = 2 * (w % NH), j0 = NH * (w / NH);   // input blocks i0, i0+1; outputs j0..
    const int unit = blockIdx.x;
    const int slice = unit / nchunks, ci = unit % nchunks;
    const size_t t0 = (size_t)slice * T + (size_t)ci * chunk;
    const int n = min(chunk, T - ci * chunk);
    const int nsteps = (n + kKStep - 1) / kKStep;

    // loader role: thread -> (token, 8-feature group) of the 32-token step
    const int lt = tid / (D / 8), lq = tid % (D / 8);
    const int lblk = ((lt >> 4) * NB + (lq >> 1)) * BLK;   // block of (token group, feature block)
    const int loff = lblk + (lt & 15) * 4 + (lq & 1) * 2;  // row (token), half (8 features)

    auto load = [&](int st, u32x4& kv, u32x4& vv, float& e) {
        const int tok = st * kKStep + lt;
        const bool live = tok < n;
        const size_t r = (t0 + (live ? tok : 0)) * D + 8 * lq;
        kv = *(const u32x4*)(K + r);
        vv = *(const u32x4*)(V + r);
        e = ETA_TOKEN ? eta[t0 + (live ? tok : 0)] : eta_scalar;
        if (!live) e = 0.f;   // padding tokens contribute nothing
        if (!live) kv = u32x4{0, 0, 0, 0};
    };
    auto scale = [&](u32x4 x, float e) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = pack_bf16x2(__uint_as_float(x[i] << 16) * e, __uint_as_float(x[i] & 0xffff0000u) * e);
        return r;
    };
    auto store = [&](int buf, u32x4 kv, u32x4 vv, float e) {
        lds[buf][TK][loff] = lo_half(kv);
        lds[buf][TK][loff + 1] = hi_half(kv);
        if (ETA_TOKEN) {
            const u32x4 ek = scale(kv, e);
            lds[buf][TEK][loff] = lo_half(ek);
            lds[buf][TEK][loff + 1] = hi_half(ek);
        }
        const u32x4 ev = ETA_TOKEN ? scale(vv, e) : vv;
        lds[buf][TV][loff] = lo_half(ev);
        lds[buf][TV][loff + 1] = hi_half(ev);
    };
    // x32 operand of feature block `fb` from tile `which`: slots 0..3 = tokens
    // 4g..4g+3, slots 4..7 = tokens 16+4g..16+4g+3
    auto operand = [&](int buf, int which, int fb) {
        auto p0 = (__attribute__((address_space(3))) s16x4*)(&lds[buf][which][fb * BLK] + lane);
        auto p1 = (__attribute__((address_space(3))) s16x4*)(&lds[buf][which][(NB + fb) * BLK] + lane);
        const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0));
        const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1));
        return u32x4{a.x, a.y, b.x, b.y};
    };

    f32x4 Pacc[2][NH], Bacc[2][NH];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) Pacc[ii][jj] = Bacc[ii][jj] = f32x4{0, 0, 0, 0};

    u32x4 kv, vv;
    float e;
    load(0, kv, vv, e);
    store(0, kv, vv, e);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const bool next = st + 1 < nsteps;
        if (next) load(st + 1, kv, vv, e);
        u32x4 aK[2], aKp[2];   // (eta K)^T and K^T of input blocks i0, i0+1
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            aKp[ii] = operand(buf, TK, i0 + ii);
            aK[ii] = ETA_TOKEN ? operand(buf, TEK, i0 + ii) : aKp[ii];
        }
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) {
            const u32x4 bK = operand(buf, TK, j0 + jj);
            const u32x4 bV = operand(buf, TV, j0 + jj);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                Pacc[ii][jj] = mfma32(aK[ii], bK, Pacc[ii][jj]);
                Bacc[ii][jj] = mfma32(aKp[ii], bV, Bacc[ii][jj]);
            }
        }
        if (next) store(buf ^ 1, kv, vv, e);
        __syncthreads();
    }

    const float sc = ETA_TOKEN ? 1.f : eta_scalar;
    uint16_t* P = Pout + (size_t)unit * D * D;
    float* B = Bout + (size_t)unit * D * D;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < NH; ++jj) {
            // lane (j', g): rows i = 16 i + 4g + r of column 16 j + j'
            const int i = i0 + ii, j = j0 + jj;
            *(u32x2*)(P + (size_t)(16 * j + c) * D + 16 * i + 4 * g) = pack_bf16x4(Pacc[ii][jj] * sc);
            *(f32x4*)(B + (size_t)(16 * j + c) * D + 16 * i + 4 * g) = Bacc[ii][jj] * sc;
        }
}

// ---------------------------------------------------------------------------
// Kernel B.  One wave per (batch*head, 16 output rows): the state rows live in
// fp32 C/D tiles as in the sub-tile kernels (lane = output row o, values = input
// features pi(jb, 4g + r)).  Per chunk: store W_c, then
//   W_{c+1}^T tile jb = W_c^T tile jb + B_c^T tile jb + P_c(rows pi(jb, .)) (-W_c)^T,
// with P_c as the A operand (rows of P, 16-byte loads) and -W_c in bf16 as B.
// The operands of the next two chunks are in flight while one is applied.
// ---------------------------------------------------------------------------
//
// With a momentum state (MOM) the chunk's negated gradient A = B_c^T - P_c W_c^T
// feeds mom^T <- beta mom^T - (1 - beta) A and W_{c+1}^T = W_c^T - mom^T, the
// momentum tiles kept in the state's layout.
template <int D, bool MOM>
__global__ __launch_bounds__(64) void bigchunk_chain_kernel(
    const float* W0, const uint16_t* __restrict__ P, const float* __restrict__ Bm,
    float* __restrict__ Wc, float* W_out, int BH, int nchunks, float beta,
    const float* __restrict__ mom0, float* __restrict__ mom_out)
{
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    const int lane = threadIdx.x;
    const int c = lane & 15, g = lane >> 4;
    int slice, ob;
    xcd_unit_part(blockIdx.x, NB, slice, ob);
    if (slice >= BH) return;
    const int out0 = 16 * ob;

    f32x4 M[NB], Mo[NB];
    {
        const float* w = W0 + (size_t)slice * D * D + (size_t)(out0 + c) * D;
        const float* mo = mom0 ? mom0 + (size_t)slice * D * D + (size_t)(out0 + c) * D : nullptr;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[2 * m] = *(const f32x4*)(w + 32 * m + 8 * g);
            M[2 * m + 1] = *(const f32x4*)(w + 32 * m + 8 * g + 4);
            if constexpr (MOM) {
                Mo[2 * m] = mo ? *(const f32x4*)(mo + 32 * m + 8 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
                Mo[2 * m + 1] =
                    mo ? *(const f32x4*)(mo + 32 * m + 8 * g + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    // operands of chunk cc: rows pi(jb, c) of P_cc, and B_cc^T tiles
    auto loadP = [&](int cc, u32x4 (&pf)[NB][NM], f32x4 (&bt)[NB]) {
        const uint16_t* Pc = P + ((size_t)slice * nchunks + cc) * D * D;
        const float* Bc = Bm + ((size_t)slice * nchunks + cc) * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int prow = 32 * (jb >> 1) + 8 * (c >> 2) + 4 * (jb & 1) + (c & 3);   // pi(jb, c)
#pragma unroll
            for (int m = 0; m < NM; ++m)
                pf[jb][m] = *(const u32x4*)(Pc + (size_t)prow * D + 32 * m + 8 * g);
            bt[jb] = *(const f32x4*)(Bc + 32 * (jb >> 1) + 8 * g + 4 * (jb & 1));
        }
    };
    // two chunks of operands in flight: ring position cc & 1, static per half of
    // the unrolled loop body
    u32x4 pf[2][NB][NM];
    f32x4 bt[2][NB];
    loadP(0, pf[0], bt[0]);
    if (nchunks > 1) loadP(1, pf[1], bt[1]);
    auto chunk_step = [&](int cc, auto rc) {
        constexpr int r = decltype(rc)::value;
        float* wc = Wc + ((size_t)slice * nchunks + cc) * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            *(f32x4*)(wc + 32 * m + 8 * g) = M[2 * m];
            *(f32x4*)(wc + 32 * m + 8 * g + 4) = M[2 * m + 1];
        }
        // -W_c in bf16 (the sign goes on the state, not on the 8x larger P operand)
        u32x4 Mn[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m)
            Mn[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]) ^
                    u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            if constexpr (MOM) {
                f32x4 acc = bt[r][jb];
#pragma unroll
                for (int m = 0; m < NM; ++m) acc = mfma32(pf[r][jb][m], Mn[m], acc);
                Mo[jb] = beta * Mo[jb] - (1.f - beta) * acc;
                M[jb] -= Mo[jb];
            } else {
                f32x4 acc = M[jb] + bt[r][jb];
#pragma unroll
                for (int m = 0; m < NM; ++m) acc = mfma32(pf[r][jb][m], Mn[m], acc);
                M[jb] = acc;
            }
        }
        if (cc + 2 < nchunks) loadP(cc + 2, pf[r], bt[r]);
    };
    int cc = 0;
    for (; cc + 2 <= nchunks; cc += 2) {
        chunk_step(cc, std::integral_constant<int, 0>{});
        chunk_step(cc + 1, std::integral_constant<int, 1>{});
    }
    if (cc < nchunks) chunk_step(cc, std::integral_constant<int, 0>{});
    float* w = W_out + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        *(f32x4*)(w + 32 * m + 8 * g) = M[2 * m];
        *(f32x4*)(w + 32 * m + 8 * g + 4) = M[2 * m + 1];
    }
    if constexpr (MOM) {
        float* mo = mom_out + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            *(f32x4*)(mo + 32 * m + 8 * g) = Mo[2 * m];
            *(f32x4*)(mo + 32 * m + 8 * g + 4) = Mo[2 * m + 1];
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel C.  One workgroup of d/16 waves per (batch*head, chunk), started from
// the chunk's stored state W_c; wave w owns output rows 16w .. 16w+15.  The chunk
// is walked in 16-token sub-tiles tau with the running matrix
//     M_tau = W_c - sum_{tau' < tau} E_tau' diag(eta) K_tau'^T :
//     E_tau = K_tau W_c^T - V_tau          (frozen chunk-start state),
//     F_tau = -diag(eta) E_tau,
//     Z_tau = Q_tau M_tau^T + (causal, inclusive Q_tau K_tau^T) F_tau,
//     M_tau+1 = M_tau + F_tau^T K_tau,
// which is the chunk's dual form with only 16 x 16 masks formed.
//
// Every wave needs the whole K and Q sub-tile.  They are loaded once per
// workgroup -- each thread fetches one 16-byte granule (coalesced, through a
// register ring eight sub-tiles deep) and stores it to a double-buffered LDS
// tile -- and every wave reads its matrix-core operands from there: row reads
// for K and Q (lane = token) and the gfx950 transpose read for K with the
// feature in the lanes.  Granules are XOR-swizzled per row so that both read
// patterns are free of bank conflicts.  One barrier per sub-tile.
// ---------------------------------------------------------------------------

// eta modes of kernel C: scalar, per-token single loads, per-token 16-byte loads
enum { kSegEtaScalar = 0, kSegEtaToken = 1, kSegEtaToken4 = 2 };

// START: the chunk-start read order, Z_tau = Q_tau W_c^T for every sub-tile (no E,
// no running M, no causal term; K, V and eta are not read).
template <int D, int ETA, bool FULL, int RB, bool START>
__global__ __launch_bounds__(4 * D / RB) void bigchunk_seg_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* __restrict__ Wstart, uint16_t* __restrict__ Z, int T, int chunk, int nseg)
{
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    constexpr int G = D / 8;           // 16-byte granules per row
    constexpr int NTH = 4 * D / RB;    // threads; each stages RB granules per sub-tile
    constexpr int P = RB == 1 ? 8 : 4; // sub-tiles in flight per thread
    __shared__ KQTile16<D> L[2];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int slice = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int t0 = seg * chunk;
    const int nc = min(chunk, T - t0);          // tokens in this chunk
    const int ntile = (nc + 15) / 16;
    const size_t tok0 = (size_t)slice * T + t0;
    const int out0 = 16 * RB * wave;            // first state row of this wave
    // token of row r of sub-tile tau, clamped into the chunk (clamped rows are
    // re-reads whose tokens get eta = 0 and no store)
    auto tok = [&](int tau, int r) {
        const int tt = tau < ntile ? tau : ntile - 1;
        const int t = 16 * tt + r;
        return FULL ? t : (t < nc ? t : nc - 1);
    };

    // this thread's granules of each staged sub-tile (K granules first, then Q)
    int which[RB], grow[RB], ggr[RB], lpos[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int gi = tid + r * NTH;
        which[r] = gi / (16 * G);
        grow[r] = (gi / G) & 15;
        ggr[r] = gi % G;
        lpos[r] = grow[r] * G + (ggr[r] ^ tile16_swizzle<D>(grow[r]));
    }
    auto gload = [&](int tau, int r) {
        if constexpr (START) {
            if (which[r] == 0) return u32x4{0u, 0u, 0u, 0u};
        }
        const uint16_t* src = which[r] ? Q : K;
        return *(const u32x4*)(src + (tok0 + tok(tau, grow[r])) * D + 8 * ggr[r]);
    };
    // this lane's V (token c, features out0 + 16 rb + 4g ..) and eta (tokens 4g ..)
    auto vload = [&](int tau, int rb) {
        if constexpr (START) return u32x2{0u, 0u};
        return *(const u32x2*)(V + (tok0 + tok(tau, c)) * D + out0 + 16 * rb + 4 * g);
    };
    auto eload = [&](int tau) {
        if constexpr (START) return f32x4{0.f, 0.f, 0.f, 0.f};
        if (ETA == kSegEtaToken4) {
            const int tt = tau < ntile ? tau : ntile - 1;
            return *(const f32x4*)(eta + tok0 + 16 * tt + 4 * g);
        } else if (ETA == kSegEtaToken) {
            f32x4 e;
#pragma unroll
            for (int r = 0; r < 4; ++r) e[r] = eta[tok0 + tok(tau, 4 * g + r)];
            return e;
        } else {
            return f32x4{eta_scalar, eta_scalar, eta_scalar, eta_scalar};
        }
    };

    // chunk-start state rows of this wave: fp32 running M and bf16 copies
    f32x4 M[RB][NB];
    u32x4 Wf[RB][NM], Mf[RB][NM];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float* w = Wstart + ((size_t)slice * nseg + seg) * D * D +
                         (size_t)(out0 + 16 * rb + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[rb][2 * m] = *(const f32x4*)(w + 32 * m + 8 * g);
            M[rb][2 * m + 1] = *(const f32x4*)(w + 32 * m + 8 * g + 4);
            Wf[rb][m] = Mf[rb][m] = pack_bf16x8(M[rb][2 * m], M[rb][2 * m + 1]);
        }
    }
    const u32x2 I16 = identity_b16(lane);

    u32x4 rg[P][RB];
    u32x2 rv[P][RB];
    f32x4 re[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            rg[p][r] = gload(p, r);
            rv[p][r] = vload(p, r);
        }
        re[p] = eload(p);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        L[0].g[which[r]][lpos[r]] = rg[0][r];
        rg[0][r] = gload(P, r);
    }
    __syncthreads();

    // 16-deep products as 32-deep ones whose upper half is zero in one operand
    // and finite in the other: these tuples live across the loop with their zero
    // halves never written, so no zeros are moved in per product
    u32x4 ktz[NB], smz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) ktz[jb] = u32x4{0u, 0u, 0u, 0u};
    const u32x4 II = {I16.x, I16.y, I16.x, I16.y};

    // one sub-tile; p = tau % P is a compile-time ring position (tau - p is a
    // multiple of the even P, so the LDS slot tau & 1 is p & 1)
    auto step = [&](int tau, auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int p1 = (p + 1) % P;
        constexpr int sl = p & 1;
        // stage the next sub-tile, refill its register slots
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (tau + 1 < ntile) L[sl ^ 1].g[which[r]][lpos[r]] = rg[p1][r];
            rg[p1][r] = gload(tau + 1 + P, r);
        }

        const u32x4* Kt = L[sl].g[0];
        const u32x4* Qt = L[sl].g[1];
        u32x4 kop[NM], qop[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int gi = c * G + ((4 * m + g) ^ tile16_swizzle<D>(c));
            if constexpr (!START) kop[m] = Kt[gi];
            qop[m] = Qt[gi];
        }
        if constexpr (START) {
            // every token of the chunk reads the chunk-start state
            const int n = FULL ? 16 : min(16, nc - 16 * tau);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                f32x4 Zt = {0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < NM; ++m) Zt = mfma32(Wf[rb][m], qop[m], Zt);
                if (FULL || c < n)
                    *(u32x2*)(Z + (tok0 + 16 * tau + c) * D + out0 + 16 * rb + 4 * g) =
                        pack_bf16x4(Zt);
            }
            __syncthreads();
            return;
        }
        // K with the feature in the lanes: supplying lane (r, q) of group g reads
        // the 8 bytes K[4g + r][32m + 8q + 4h .. +3] of block jb = 2m + h
        // (upper halves of ktz: [0 | K^T] [I ; F] = K^T F)
        {
            const int r = (lane >> 2) & 3, q = lane & 3;
            const int row = 4 * g + r;
            const u32x2* base = reinterpret_cast<const u32x2*>(Kt) + row * (2 * G);
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                const int m = jb >> 1, h = jb & 1;
                auto pt = (__attribute__((address_space(3))) s16x4*)(
                    base + 2 * ((4 * m + q) ^ tile16_swizzle<D>(row)) + h);
                const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(pt));
                ktz[jb].z = t.x;
                ktz[jb].w = t.y;
            }
        }
        const int n = FULL ? 16 : min(16, nc - 16 * tau);
        f32x4 et = re[p];
        if (!FULL) {
            et.x = (4 * g + 0 < n) ? et.x : 0.f;
            et.y = (4 * g + 1 < n) ? et.y : 0.f;
            et.z = (4 * g + 2 < n) ? et.z : 0.f;
            et.w = (4 * g + 3 < n) ? et.w : 0.f;
        }
        // causal scores S[s][t] = k_s . q_t for s <= t (shared by the row blocks)
        f32x4 St = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NM; ++m) St = mfma32(kop[m], qop[m], St);
        f32x4 Sm;
        Sm.x = (4 * g + 0 <= c) ? St.x : 0.f;
        Sm.y = (4 * g + 1 <= c) ? St.y : 0.f;
        Sm.z = (4 * g + 2 <= c) ? St.z : 0.f;
        Sm.w = (4 * g + 3 <= c) ? St.w : 0.f;
        {
            const u32x2 Sb = pack_bf16x4(Sm);
            smz.z = Sb.x;
            smz.w = Sb.y;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            // E = K W_c^T - V (tokens in the rows, this block's outputs in the lanes)
            {
                const u32x2 vneg = rv[p][rb] ^ u32x2{0x80008000u, 0x80008000u};
                vz.x = vneg.x;
                vz.y = vneg.y;
            }
            f32x4 Et = mfma32(vz, II, f32x4{0, 0, 0, 0});   // [-V | 0] [I ; I]
#pragma unroll
            for (int m = 0; m < NM; ++m) Et = mfma32(kop[m], Wf[rb][m], Et);
            const u32x2 F = pack_bf16x4(-et * Et);
            const u32x4 IF = {I16.x, I16.y, F.x, F.y};
            // Z = Q M^T + S^T-weighted F (outputs in the rows, tokens in the lanes)
            f32x4 Zt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Zt = mfma32(Mf[rb][m], qop[m], Zt);
            Zt = mfma32(IF, smz, Zt);   // + [I | F^T] [0 ; scores]
            if (FULL || c < n)
                *(u32x2*)(Z + (tok0 + 16 * tau + c) * D + out0 + 16 * rb + 4 * g) =
                    pack_bf16x4(Zt);
            // M += F^T K
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) M[rb][jb] = mfma32(ktz[jb], IF, M[rb][jb]);
#pragma unroll
            for (int m = 0; m < NM; ++m) Mf[rb][m] = pack_bf16x8(M[rb][2 * m], M[rb][2 * m + 1]);
            rv[p][rb] = vload(tau + P, rb);
        }
        re[p] = eload(tau + P);
        __syncthreads();
    };

    int tau0 = 0;
    for (; tau0 + P <= ntile; tau0 += P) {
        step(tau0 + 0, std::integral_constant<int, 0>{});
        step(tau0 + 1, std::integral_constant<int, 1>{});
        step(tau0 + 2, std::integral_constant<int, 2>{});
        step(tau0 + 3, std::integral_constant<int, 3>{});
        if constexpr (P == 8) {
            step(tau0 + 4, std::integral_constant<int, 4 % P>{});
            step(tau0 + 5, std::integral_constant<int, 5 % P>{});
            step(tau0 + 6, std::integral_constant<int, 6 % P>{});
            step(tau0 + 7, std::integral_constant<int, 7 % P>{});
        }
    }
    if (tau0 + 0 < ntile) step(tau0 + 0, std::integral_constant<int, 0>{});
    if (tau0 + 1 < ntile) step(tau0 + 1, std::integral_constant<int, 1>{});
    if (tau0 + 2 < ntile) step(tau0 + 2, std::integral_constant<int, 2>{});
    if constexpr (P == 8) {
        if (tau0 + 3 < ntile) step(tau0 + 3, std::integral_constant<int, 3>{});
        if (tau0 + 4 < ntile) step(tau0 + 4, std::integral_constant<int, 4 % P>{});
        if (tau0 + 5 < ntile) step(tau0 + 5, std::integral_constant<int, 5 % P>{});
        if (tau0 + 6 < ntile) step(tau0 + 6, std::integral_constant<int, 6 % P>{});
    }
}


template <int D, int ETA, bool FULL, bool START = false>
void launch_seg(const LinearArgs& a, const float* Wc, int nchunks, hipStream_t s)
{
    // two 16-row state blocks per wave: one wave per SIMD, each K/Q operand and
    // score serving both blocks
    constexpr int RB = 2;
    hipLaunchKernelGGL((bigchunk_seg_kernel<D, ETA, FULL, RB, START>),
                       dim3((unsigned)(a.BH * nchunks)),
                       dim3(4 * D / RB), 0, s, (const uint16_t*)a.K, (const uint16_t*)a.Q,
                       (const uint16_t*)a.V, a.eta, a.eta_scalar, Wc, (uint16_t*)a.Z, a.T, a.chunk,
                       nchunks);
}

template <int D>
hipError_t launch_d(const LinearArgs& a, hipStream_t s)
{
    const int nchunks = (a.T + a.chunk - 1) / a.chunk;
    const size_t mats = (size_t)a.BH * nchunks * D * D;
    uint16_t* P = (uint16_t*)a.workspace;
    float* Bm = (float*)((char*)a.workspace + mats * sizeof(uint16_t));
    float* Wc = Bm + mats;

    if (a.eta)
        hipLaunchKernelGGL((bigchunk_gram_kernel<D, true>), dim3((unsigned)(a.BH * nchunks)),
                           dim3(64 * (D / 16)), 0, s, (const uint16_t*)a.K, (const uint16_t*)a.V,
                           a.eta, a.eta_scalar, P, Bm, a.T, a.chunk, nchunks);
    else
        hipLaunchKernelGGL((bigchunk_gram_kernel<D, false>), dim3((unsigned)(a.BH * nchunks)),
                           dim3(64 * (D / 16)), 0, s, (const uint16_t*)a.K, (const uint16_t*)a.V,
                           a.eta, a.eta_scalar, P, Bm, a.T, a.chunk, nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int units = (a.BH + 7) / 8 * 8;
    if (a.momentum)
        hipLaunchKernelGGL((bigchunk_chain_kernel<D, true>), dim3((unsigned)(units * (D / 16))),
                           dim3(64), 0, s, a.W0, P, Bm, Wc, a.W_out, a.BH, nchunks, a.beta, a.mom0,
                           a.mom_out);
    else
        hipLaunchKernelGGL((bigchunk_chain_kernel<D, false>), dim3((unsigned)(units * (D / 16))),
                           dim3(64), 0, s, a.W0, P, Bm, Wc, a.W_out, a.BH, nchunks, 0.f, nullptr,
                           nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // every sub-tile full: T (and the chunk, a multiple of 32) divide into 16s
    const bool full = a.T % 16 == 0;
    const bool eta4 = a.eta && full && reinterpret_cast<uintptr_t>(a.eta) % 16 == 0;
    if (a.read_start) {
        if (full) launch_seg<D, kSegEtaScalar, true, true>(a, Wc, nchunks, s);
        else launch_seg<D, kSegEtaScalar, false, true>(a, Wc, nchunks, s);
    } else if (full) {
        if (!a.eta) launch_seg<D, kSegEtaScalar, true>(a, Wc, nchunks, s);
        else if (eta4) launch_seg<D, kSegEtaToken4, true>(a, Wc, nchunks, s);
        else launch_seg<D, kSegEtaToken, true>(a, Wc, nchunks, s);
    } else {
        if (!a.eta) launch_seg<D, kSegEtaScalar, false>(a, Wc, nchunks, s);
        else launch_seg<D, kSegEtaToken, false>(a, Wc, nchunks, s);
    }
    return hipGetLastError();
}

}  // namespace

bool linear_bigchunk_supported(int d, int chunk, int bf16)
{
    return bf16 && (d == 64 || d == 128) && chunk >= 128 && chunk % kKStep == 0;
}

size_t linear_bigchunk_workspace(int BH, int T, int d, int chunk)
{
    const size_t nchunks = ((size_t)T + chunk - 1) / chunk;
    const size_t mats = (size_t)BH * nchunks * d * d;
    return mats * (sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t launch_linear_bigchunk(const LinearArgs& a, hipStream_t s)
{
    switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ttt
