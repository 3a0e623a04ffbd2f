// TTT-Linear forward scan, chunks of 16 tokens, for few (batch, head) slices
// with long sequences: the sequence of every slice is cut into S segments so
// that S * slices workgroups fill the compute units.
//
// The chunk map is affine in the state: W -> W (I - P_c) + B_c with
// P_c = K_c^T diag(eta) K_c, B_c = V_c^T diag(eta) K_c (PaperTrace "5 · TestingTime
// 训练与长上下文" §1.1/§2.3; the dual form of diosapp "Test-Time Training (TTT)
// guide" §3 inside a chunk), so the end state of segment k is W_B,k + W_start,k A_k,
// where A_k is the product of the segment's (I - P_c) and W_B,k its end state
// from zero.  Three launches:
//   pass 1   segment 0 scans from W0 (Z written, end state kept); segments
//            1 .. S-1 form their maps (W_B, A), reading their chunks backwards:
//            one chain per wave (A^T) and W_B accumulated beside it, no Z;
//   combine  W_start,1 = end of segment 0, W_start,k+1 = W_B,k + W_start,k A_k;
//   pass 2   segments 1 .. S-1 scan again from W_start,k (Z written; the last
//            one's end state is W_T).
// Every token is read twice past segment 0 (once for the map, once for the
// replay), but no chain is longer than the longest segment.
//
// A workgroup is one (slice, segment) on one compute unit: four waves, wave w
// owning state rows 16w .. 16w+15, sharing each chunk's K, Q and V through a
// ring of LDS tiles.  One unit's vector-memory path, not the matrix cores, bounds
// a chunk step, and its cost follows the cache lines an instruction touches more
// than the bytes: every global access is a contiguous piece per wave (K and Q in
// 16-byte granules, V and Z in 8-byte pieces, 512 bytes per wave), never the
// 16-row stripe of one wave's features.  Z goes out through LDS one group of
// chunks later, after the barrier that makes all four waves' parts visible.
// Per-token eta is read per lane (the four tokens of its rows, one 16-byte load
// with few distinct lines); staging it through LDS measured slower.
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"
#include "mfma_f32.h"

namespace ttt {
namespace {

enum { kSegScan = 0, kSegMap = 1 };
enum { kSegEtaScalar = 0, kSegEtaToken = 1, kSegEtaToken4 = 2 };

typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kSegD = 64;

template <typename F, int... I>
__device__ __forceinline__ void seg_unroll(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

// Where the segments of a slice start: segment 0 holds n0 chunks, the others n1
// each (the last one takes what is left), all whole 16-token chunks.
struct SegPlan {
    int S;       // segments per slice
    int n0, n1;  // chunks of segment 0 and of the middle segments
    int nch;     // chunks of the whole sequence
};

__host__ __device__ inline int seg_first_chunk(const SegPlan& p, int k)
{
    return k == 0 ? 0 : p.n0 + (k - 1) * p.n1;
}

__host__ __device__ inline int seg_chunks(const SegPlan& p, int k)
{
    return k == 0 ? p.n0 : (k == p.S - 1 ? p.nch - p.n0 - (p.S - 2) * p.n1 : p.n1);
}

// Workspace, per slice: W_B, A and W_start of every segment (index 0 of W_start
// holding segment 0's end state), [D, D] fp32 each.
struct SegWorkspace {
    float* wb;      // [BH, S, D, D]
    float* amap;    // [BH, S, D, D]
    float* wstart;  // [BH, S, D, D]
};

__host__ __device__ inline SegWorkspace seg_workspace(void* base, int BH, int S)
{
    SegWorkspace w;
    const size_t n = (size_t)BH * S * kSegD * kSegD;
    w.wb = reinterpret_cast<float*>(base);
    w.amap = w.wb + n;
    w.wstart = w.amap + n;
    return w;
}

// chunks per barrier, chunks staged ahead, LDS ring slots (as the many-head
// kernel with four waves)
constexpr int kSegGroup = 4;
constexpr int kSegAhead = 2 * kSegGroup;
constexpr int kSegSlots = 2 * kSegAhead;

// One chunk's inputs in LDS.  K and Q (a map: K and V) as swizzled 16-byte
// granules (row operand and transposed reads conflict-free within a 16-lane
// group).  A scan's V as 8-byte units (four features), unit u of token r at
// r * 16 + (u ^ seg_vswz(r)): the 16 tokens a lane group reads at one unit then
// fall on distinct banks.
struct SegTile {
    u32x4 g[2][16 * (kSegD / 8)];
    u32x2 v[16 * 16];
};

__device__ __forceinline__ int seg_vswz(int r) { return (r >> 1) & 7; }

// Z of a group of chunks waits in LDS (same unit layout as V) until the barrier
// that ends the group; two groups alternate.
typedef u32x2 SegZStage[2 * kSegGroup][16 * 16];

// A raw buffer store at or past the resource's size is dropped by the memory unit.
constexpr int kSegBufferFlags = 0x00020000;   // dword 3 of a gfx9 buffer resource: raw 32-bit data
constexpr int kSegDropOffset = 0x7ffffff0;
// Cache policy of the accesses whose bytes a workgroup touches once and no later
// pass reads again (a scan's K, Q and V, every Z store): the non-temporal bit of
// gfx950's cache-policy operand, so that they do not push out of the caches the K
// and V tiles that pass 1's maps read and pass 2 reads again.  eta keeps the
// default policy: all four waves read each of its lines.  Per call at 1 x 32
// heads, T = 32768: 166 -> 155 us.
constexpr int kSegStream = 2;

// One (slice, segment) on a workgroup of four waves.
//   SCAN: from the segment's start state (W0 for segment 0, else W_start), Z
//         written; the end state goes to W_out for the last segment, to
//         W_start[0] for segment 0.
//   MAP:  the segment's chunks in reverse order.  P_c is symmetric, so the
//         suffix products R_c = (I - P_c) R_{c+1} (R_{n+1} = I, R_1 = A) satisfy
//         R_c^T = R_{c+1}^T (I - P_c): the scan recurrence without V, run on the
//         rows of R^T from the identity.  Beside it, with no feedback into the
//         chain, W_B = sum_c B_c R_{c+1} = sum_c V_c^T diag(eta) (K_c R_{c+1}),
//         K_c R_{c+1} being the chain's own E for chunk c.  Both leave transposed
//         back through LDS.  Reading the segment backwards also means its first
//         chunks are the last ones pass 1 reads, the first ones pass 2 replays.
// RAG: the last segment of a sequence whose length is not a multiple of 16 (a
// scan, pass 2 only).  Its K, Q, V and eta come through range-checked buffer
// resources over the segment's rows (the whole offset in the vector offset, the
// part the check covers), so rows past T, and steps past the end, read as zero;
// a zero row of K and V gives a zero row of E, hence of F, so such a token adds
// nothing, whatever its eta.  Z rows past T fall outside Z's resource.
template <int MODE, int ETA, bool RAG = false>
__device__ __forceinline__ void seg_body(
    SegTile* L, SegZStage& Zs, const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, void* ws, int BH, int T,
    const SegPlan& plan, int slice, int seg)
{
    constexpr bool MAP = MODE == kSegMap;
    constexpr int D = kSegD;
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    constexpr int G = D / 8;           // 16-byte granules per row
    constexpr int kGroup = kSegGroup;
    constexpr int P = kSegAhead;
    constexpr int kSlots = kSegSlots;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int ch0 = seg_first_chunk(plan, seg);
    const int nch = seg_chunks(plan, seg);
    const size_t tok0 = (size_t)slice * T + (size_t)16 * ch0;
    const int out0 = 16 * wave;
    const SegWorkspace w = seg_workspace(ws, BH, plan.S);
    const size_t dd = (size_t)D * D;
    const size_t sw = ((size_t)slice * plan.S + seg) * dd;   // this segment's [D, D] block

    // Every wave issues the same loads (a wave-dependent load count would make the
    // compiler wait on the prefetch ring early).  Threads 0..127 load a 16-byte
    // granule of K, threads 128..255 one of Q (scan) or of V (map), into the tile's
    // second granule array; a scan also loads V as one 8-byte piece per thread.
    constexpr bool kV8 = !MAP;
    const int which = tid / (16 * G);
    const int grow = (tid / G) & 15;
    const int ggr = tid % G;
    const int lpos = grow * G + (ggr ^ tile16_swizzle<D>(grow));
    // first token of the chunk that step ch processes (steps past the end re-read
    // the last one)
    auto chunk_base = [&](int ch) {
        const int cc = ch < nch ? ch : nch - 1;
        return tok0 + (size_t)16 * (MAP ? nch - 1 - cc : cc);
    };
    // thread t's 8-byte piece of a V (or Z) tile: token t / 16, unit t % 16
    const int vrow = tid >> 4;
    const int vpos = vrow * 16 + ((tid & 15) ^ seg_vswz(vrow));
    // this lane's unit of a V (or Z) tile: token c, features out0 + 4g .. out0 + 4g + 3
    const int opos = c * 16 + ((4 * wave + g) ^ seg_vswz(c));
    // RAG: the segment's rows [tok0, slice start + T) as buffer resources
    static_assert(!(RAG && MAP), "only a scan takes the ragged form");
    const int rows = RAG ? T - 16 * ch0 : 0;
    auto rsrc = [](const void* base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kSegBufferFlags);
    };
    const auto bK = rsrc(K + tok0 * D, rows * D * 2), bQ = rsrc(Q + tok0 * D, rows * D * 2);
    const auto bV = rsrc(V + tok0 * D, rows * D * 2);
    const auto bE = rsrc(eta ? eta + tok0 : nullptr, eta ? rows * 4 : 0);
    auto gload = [&](u32x4& r, int ch) {
        if constexpr (RAG) {   // wave >> 1 == which, uniform
            r = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                (wave >> 1) ? bQ : bK, (16 * ch + grow) * (2 * D) + 16 * ggr, 0, kSegStream));
        } else {
            const uint16_t* src = which ? (MAP ? V : Q) : K;
            const u32x4* p = (const u32x4*)(src + chunk_base(ch) * D + (grow * D + 8 * ggr));
            if constexpr (MAP) r = *p;   // read again by pass 2's replay
            else r = __builtin_nontemporal_load(p);
        }
    };
    auto vload = [&](int ch) {
        if constexpr (RAG)
            return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                bV, (16 * ch * D + 4 * tid) * 2, 0, kSegStream));
        else   // a scan's V (the maps take V through gload)
            return __builtin_nontemporal_load((const u32x2*)(V + chunk_base(ch) * D + 4 * tid));
    };
    // eta of tokens 4g .. 4g + 3 (the rows of this lane's E tile)
    auto eload = [&](int ch) {
        if constexpr (ETA == kSegEtaToken4 && RAG) {
            return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                bE, (16 * ch + 4 * g) * 4, 0, 0));
        } else if constexpr (ETA == kSegEtaToken4) {
            return *(const f32x4*)(eta + chunk_base(ch) + 4 * g);
        } else if constexpr (ETA == kSegEtaToken) {
            f32x4 e;
            if constexpr (RAG) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    e[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        bE, (16 * ch + 4 * g + r) * 4, 0, 0));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = eta[chunk_base(ch) + 4 * g + r];
            }
            return e;
        } else {
            return f32x4{eta_scalar, eta_scalar, eta_scalar, eta_scalar};
        }
    };
    auto stage = [&](SegTile& t, const u32x4& r, const u32x2& v) {
        t.g[which][lpos] = r;
        if constexpr (kV8) t.v[vpos] = v;
    };
    // -V of the chunk in slot t for the scan's E (the map's chain has no V)
    auto vneg = [&](const SegTile& t) {
        if constexpr (MAP) return u32x2{0u, 0u};
        else return t.v[opos] ^ u32x2{0x80008000u, 0x80008000u};
    };
    // Z of chunk ch as thread tid's piece, dropped for ch < 0 (and rows past T)
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(Z + tok0 * D, 0,
                                                      (RAG ? rows : nch * 16) * D * 2,
                                                      kSegBufferFlags);
    auto zstore = [&](const u32x2& v, int ch) {
        const int off = ch >= 0 ? (ch * 16 * D + 4 * tid) * 2 : kSegDropOffset;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), rz, off, 0, kSegStream);
    };
    auto row_operand = [&](const u32x4* t, u32x4 (&op)[NM]) {
#pragma unroll
        for (int m = 0; m < NM; ++m) op[m] = t[c * G + ((4 * m + g) ^ tile16_swizzle<D>(c))];
    };
    // the tile's transpose, features 16 jb .. 16 jb + 15 in the lanes and the
    // chunk's tokens in the upper half of zero-padded operands
    auto trans_operand = [&](const u32x4* t, u32x4 (&op)[NB]) {
        const int r = (lane >> 2) & 3, q = lane & 3;
        const int row = 4 * g + r;
        const u32x2* base = reinterpret_cast<const u32x2*>(t) + row * (2 * G);
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            auto pt = (__attribute__((address_space(3))) s16x4*)(
                base + 2 * ((4 * (jb >> 1) + q) ^ tile16_swizzle<D>(row)) + (jb & 1));
            const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(pt));
            op[jb].z = v.x;
            op[jb].w = v.y;
        }
    };

    // state rows out0 + c, columns pi(jb, 4g + i) = 32 (jb / 2) + 8g + 4 (jb % 2) + i
    f32x4 M[NB];
    if constexpr (MAP) {
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int base = 32 * (jb >> 1) + 8 * g + 4 * (jb & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) M[jb][i] = (base + i == out0 + c) ? 1.f : 0.f;
        }
    } else {
        const float* w0 = seg == 0 ? W0 + (size_t)slice * dd : w.wstart + sw;
        const float* wr = w0 + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[2 * m] = *(const f32x4*)(wr + 32 * m + 8 * g);
            M[2 * m + 1] = *(const f32x4*)(wr + 32 * m + 8 * g + 4);
        }
    }
    u32x4 Mf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
    const u32x2 I16 = identity_b16(lane);
    // map: minus W_B, output features pi(ob, 4g + i), columns out0 + c (the
    // transposed V operand orders its features as the state's columns)
    f32x4 Sb[MAP ? NB : 1];
#pragma unroll
    for (int ob = 0; ob < (MAP ? NB : 1); ++ob) Sb[ob] = f32x4{0, 0, 0, 0};

    // step X uses LDS slot X % kSlots; tiles of steps 0 .. P-1 are stored up
    // front, and during step ch the tile of step ch + P is stored and the pieces
    // of step ch + 2P loaded (into the register slots they came from).  re[]
    // holds eta of steps ch .. ch + P - 1.
    u32x4 rg[P];
    u32x2 rv[kV8 ? P : 1] = {};
    f32x4 re[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        gload(rg[p], p);
        if constexpr (kV8) rv[p] = vload(p);
    }
    // the loads that stay in flight into the loop, in the order a step issues
    // them, so that the loop's waits count them as in the steady state
#pragma unroll
    for (int p = 0; p < P; ++p) {
        stage(L[p], rg[p], rv[kV8 ? p : 0]);
        gload(rg[p], P + p);
        if constexpr (kV8) rv[p] = vload(P + p);
        re[p] = eload(p);
    }
    __syncthreads();

    // E of the first step = K W^T (- V); kb[ch & 1] holds K of step ch as row
    // operand, the other set K of step ch + 1
    u32x4 kb[2][NM];
    row_operand(L[0].g[0], kb[0]);
    row_operand(L[1].g[0], kb[1]);
    f32x4 Et = mfma16(vneg(L[0]), I16, f32x4{0, 0, 0, 0});
#pragma unroll
    for (int m = 0; m < NM; ++m) Et = mfma32(kb[0][m], Mf[m], Et);
    // 16-deep products as 32-deep ones whose lower half is zero in one operand
    u32x4 ktz[NB], vtz[MAP ? NB : 1], smz = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) ktz[jb] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int jb = 0; jb < (MAP ? NB : 1); ++jb) vtz[jb] = u32x4{0u, 0u, 0u, 0u};

    auto step = [&](int ch, auto kc_) {
        constexpr int k = decltype(kc_)::value;
        constexpr int p = k % P;
        constexpr int j = k % kGroup;              // step within its group
        constexpr int zb = (k / kGroup) & 1;       // group parity (c0 is a multiple of 16)
        // staged unconditionally: past the end the slot receives a re-read of the last
        // chunk (read only by the unused lookahead), and a conditional use would let
        // the compiler sink the prefetch loads into the branch
        stage(L[(k + P) % kSlots], rg[p], rv[kV8 ? p : 0]);
        gload(rg[p], ch + 2 * P);
        if constexpr (kV8) rv[p] = vload(ch + 2 * P);
        // the previous group's Z, complete since the last barrier
        u32x2 zprev = {0u, 0u};
        if constexpr (!MAP) zprev = Zs[(zb ^ 1) * kGroup + j][vpos];

        constexpr int pe = p & 1;
        u32x4 (&kc)[NM] = kb[pe];
        u32x4 (&kn)[NM] = kb[pe ^ 1];
        // K with the feature in the lanes (A operand of the state update)
        trans_operand(L[k].g[0], ktz);
        const f32x4 et = re[p];
        // F = -diag(eta) E
        const u32x2 F = pack_bf16x4(-et * Et);
        const u32x4 IF = {I16.x, I16.y, F.x, F.y};
        // E of the next step = K' W^T + [-V' | G] [I ; F]  (G = K' K^T)
        {
            f32x4 Gt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Gt = mfma32(kc[m], kn[m], Gt);
            const u32x2 Gb = pack_bf16x4(Gt);
            f32x4 Pt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Pt = mfma32(kn[m], Mf[m], Pt);
            const u32x2 vn = vneg(L[(k + 1) % kSlots]);
            Et = mfma32(u32x4{vn.x, vn.y, Gb.x, Gb.y}, IF, Pt);
        }
        // W += F^T K
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) M[jb] = mfma32(ktz[jb], IF, M[jb]);
        if constexpr (MAP) {
            // -W_B += V^T F  (V with the feature in the lanes)
            trans_operand(L[k].g[1], vtz);
#pragma unroll
            for (int ob = 0; ob < NB; ++ob) Sb[ob] = mfma32(vtz[ob], IF, Sb[ob]);
        } else {
            // Z = Q W^T + causal scores times F
            u32x4 qc[NM];
            row_operand(L[k].g[1], qc);
            f32x4 St = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) St = mfma32(kc[m], qc[m], St);
            f32x4 Sm;
            Sm.x = (4 * g + 0 <= c) ? St.x : 0.f;
            Sm.y = (4 * g + 1 <= c) ? St.y : 0.f;
            Sm.z = (4 * g + 2 <= c) ? St.z : 0.f;
            Sm.w = (4 * g + 3 <= c) ? St.w : 0.f;
            f32x4 Zt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Zt = mfma32(Mf[m], qc[m], Zt);
            const u32x2 sb = pack_bf16x4(Sm);
            smz.z = sb.x;
            smz.w = sb.y;
            Zt = mfma32(IF, smz, Zt);
            Zs[zb * kGroup + j][opos] = pack_bf16x4(Zt);
            zstore(zprev, ch - kGroup);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
        row_operand(L[(k + 2) % kSlots].g[0], kc);   // K of step ch + 2 (stale past the end)
        re[p] = eload(ch + P);
        if (j == kGroup - 1) __syncthreads();
    };

    int c0 = 0;
    for (; c0 + kSlots <= nch; c0 += kSlots)
        seg_unroll([&](auto k) { step(c0 + k, k); }, std::make_integer_sequence<int, kSlots>{});
    seg_unroll([&](auto k) {
        if (c0 + k < nch) step(c0 + k, k);
    }, std::make_integer_sequence<int, kSlots - 1>{});

    if constexpr (MAP) {
        // A (= R_1, from the rows of R_1^T held here) and W_B, transposed through
        // LDS (row stride D + 1) and stored row-major
        __syncthreads();   // every wave is done with the ring
        float* ta = reinterpret_cast<float*>(L);
        float* tb = ta + D * (D + 1);
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int base = 32 * (jb >> 1) + 8 * g + 4 * (jb & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ta[(base + i) * (D + 1) + out0 + c] = M[jb][i];
                tb[(base + i) * (D + 1) + out0 + c] = -Sb[jb][i];
            }
        }
        __syncthreads();
        const int r = tid >> 2, cb = 16 * (tid & 3);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 a, b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = ta[r * (D + 1) + cb + 4 * q + i];
                b[i] = tb[r * (D + 1) + cb + 4 * q + i];
            }
            *(f32x4*)(w.amap + sw + (size_t)r * D + cb + 4 * q) = a;
            *(f32x4*)(w.wb + sw + (size_t)r * D + cb + 4 * q) = b;
        }
    } else {
        // Z of the last group and the rest of the group before it
        __syncthreads();
        const int gl = (nch - 1) / kGroup, m = nch - gl * kGroup;
        if (gl > 0)
            for (int jj = m; jj < kGroup; ++jj)
                zstore(Zs[((gl - 1) & 1) * kGroup + jj][vpos], (gl - 1) * kGroup + jj);
        for (int jj = 0; jj < m; ++jj) zstore(Zs[(gl & 1) * kGroup + jj][vpos], gl * kGroup + jj);
        // end state
        float* dst = seg == plan.S - 1 ? W_out + (size_t)slice * dd
                                       : w.wstart + ((size_t)slice * plan.S) * dd;   // segment 0
        float* wr = dst + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m2 = 0; m2 < NM; ++m2) {
            *(f32x4*)(wr + 32 * m2 + 8 * g) = M[2 * m2];
            *(f32x4*)(wr + 32 * m2 + 8 * g + 4) = M[2 * m2 + 1];
        }
    }
}

// Pass 1: workgroup (slice, segment) for segments 0 .. S-2, segment 0 scanning
// and the others forming their maps, all at once (no start state depends on the
// last segment's map, so it is never formed).  Pass 2: segments 1 .. S-1 scanning
// from their start states.  Either pass runs S - 1 workgroups per slice, and the
// segments of a slice are adjacent workgroups.
template <int ETA>
__global__ __launch_bounds__(256) void linear_seg_pass1_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, void* ws, int BH, int T,
    SegPlan plan)
{
    __shared__ SegTile L[kSegSlots];
    __shared__ SegZStage Zs;
    const int slice = (int)blockIdx.x / (plan.S - 1), seg = (int)blockIdx.x % (plan.S - 1);
    if (seg == 0)
        seg_body<kSegScan, ETA>(L, Zs, K, Q, V, eta, eta_scalar, W0, Z, W_out, ws, BH, T, plan,
                                slice, 0);
    else
        seg_body<kSegMap, ETA>(L, Zs, K, Q, V, eta, eta_scalar, W0, Z, W_out, ws, BH, T, plan,
                               slice, seg);
}

template <int ETA, bool RAGGED>
__global__ __launch_bounds__(256) void linear_seg_pass2_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, void* ws, int BH, int T,
    SegPlan plan)
{
    __shared__ SegTile L[kSegSlots];
    __shared__ SegZStage Zs;
    const int slice = (int)blockIdx.x / (plan.S - 1), seg = 1 + (int)blockIdx.x % (plan.S - 1);
    if (RAGGED && seg == plan.S - 1)
        seg_body<kSegScan, ETA, RAGGED>(L, Zs, K, Q, V, eta, eta_scalar, W0, Z, W_out, ws, BH, T,
                                        plan, slice, seg);
    else
        seg_body<kSegScan, ETA>(L, Zs, K, Q, V, eta, eta_scalar, W0, Z, W_out, ws, BH, T, plan,
                                slice, seg);
}

// W_start,k+1 = W_B,k + W_start,k A_k for k = 1 .. S-2 (W_start,1 = the end of
// segment 0, left in W_start[0] by pass 1), in fp32 on the fp32 matrix cores
// (16x16x4 products of fp32 operands): one workgroup per (slice, 16 rows), wave w
// computing columns 16w .. 16w + 15.  The current rows sit in LDS; the next map's
// A block and W_B rows load while a step computes, so the chain of S - 2 steps
// waits on memory once.  (The FMA loop over LDS this replaces took 12-13 us at
// 32 heads of 8 segments.)
__global__ __launch_bounds__(256) void seg_combine_kernel(void* ws, int BH, int S)
{
    constexpr int D = kSegD;
    constexpr int STRIDE = D + 4;   // RL reads of 16 lanes on distinct banks
    __shared__ __align__(16) float cur[16 * STRIDE];
    const SegWorkspace w = seg_workspace(ws, BH, S);
    const size_t dd = (size_t)D * D;
    const int slice = blockIdx.x, i0 = 16 * blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    float* base = w.wstart + (size_t)slice * S * dd;
    {   // W_start,1: thread tid copies 4 values of the 16 rows
        const int r = tid >> 4, q = tid & 15;
        const size_t off = (size_t)(i0 + r) * D + 4 * q;
        const f32x4 v = *(const f32x4*)(base + off);
        *(f32x4*)(base + dd + off) = v;
        *(f32x4*)(cur + r * STRIDE + 4 * q) = v;
    }
    // CL forms: a[kb] of A_k rows 16 kb .. + 15, columns 16w .. + 15; wb of W_B,k
    // rows i0 .. i0 + 15, the same columns
    f32x4 a[4], wb;
    auto fetch = [&](int k) {
        const float* ak = w.amap + ((size_t)slice * S + k) * dd;
        const float* bk = w.wb + ((size_t)slice * S + k) * dd;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) a[kb][v] = ak[(size_t)(16 * kb + 4 * g + v) * D + 16 * wave + c];
#pragma unroll
        for (int v = 0; v < 4; ++v) wb[v] = bk[(size_t)(i0 + 4 * g + v) * D + 16 * wave + c];
    };
    if (S > 2) fetch(1);
    __syncthreads();
    for (int k = 1; k + 1 < S; ++k) {
        f32x4 acc = wb;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mm16(rl<STRIDE>(cur, 16 * kb, lane), a[kb], acc);
        if (k + 2 < S) fetch(k + 1);
        __syncthreads();   // every wave has read the current rows
        put_cl<STRIDE>(cur, 16 * wave, lane, acc);
        float* dst = base + (size_t)(k + 1) * dd + (size_t)(i0 + 4 * g) * D + 16 * wave + c;
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[(size_t)v * D] = acc[v];
        __syncthreads();
    }
}

// Segment lengths: n0 = kSegFirstRatio n1.  Segment 0 scans while the others form
// their maps, so the ratio balances a scan step against a map step.  Measured per
// call (32 heads of 32768 tokens, same inputs repeated): 0.3 -> 0.181 ms, 0.4 ->
// 0.176, 0.55 -> 0.172-0.176, 0.7 -> 0.174, 0.85 -> 0.180; 16 heads: 0.55 -> 0.103,
// 0.85 -> 0.108; 8 heads of 65536: flat from 0.4 to 0.7 (0.126-0.127 ms).
constexpr double kSegFirstRatio = 0.55;
constexpr int kSegMinChunks = 32;     // shortest middle segment
constexpr int kSegUnits = 256;        // MI355X compute units

SegPlan seg_plan(int BH, int T)
{
    SegPlan p;
    p.nch = (T + 15) / 16;   // the last segment holds a partial chunk
    // S - 1 workgroups per slice in either pass, one per compute unit
    int S = kSegUnits / (BH > 0 ? BH : 1) + 1;
    S = S > 64 ? 64 : S;
    while (S > 2 && p.nch < (int)((S - 1 + kSegFirstRatio) * kSegMinChunks)) --S;
    p.S = S < 2 ? 2 : S;
    p.n1 = (int)(p.nch / (p.S - 1 + kSegFirstRatio));
    p.n0 = p.nch - (p.S - 1) * p.n1;   // the remainder goes to segment 0
    return p;
}

template <int ETA>
hipError_t launch_seg_eta(const LinearArgs& a, hipStream_t s)
{
    const SegPlan p = seg_plan(a.BH, a.T);
    const unsigned bh = (unsigned)a.BH;
    hipLaunchKernelGGL((linear_seg_pass1_kernel<ETA>), dim3(bh * (p.S - 1)), dim3(256), 0, s,
                       (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta,
                       a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.workspace, a.BH, a.T, p);
    hipLaunchKernelGGL(seg_combine_kernel, dim3(bh, kSegD / 16), dim3(256), 0, s, a.workspace,
                       a.BH, p.S);
    if (a.T % 16 == 0)
        hipLaunchKernelGGL((linear_seg_pass2_kernel<ETA, false>), dim3(bh * (p.S - 1)), dim3(256),
                           0, s, (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V,
                           a.eta, a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.workspace, a.BH,
                           a.T, p);
    else
        hipLaunchKernelGGL((linear_seg_pass2_kernel<ETA, true>), dim3(bh * (p.S - 1)), dim3(256),
                           0, s, (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V,
                           a.eta, a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.workspace, a.BH,
                           a.T, p);
    return hipGetLastError();
}

}  // namespace

bool linear_seg_supported(int BH, int T, int d, int chunk, int bf16)
{
    // at least four workgroups per slice in each pass; Z of one segment is
    // addressed by a 32-bit byte offset
    return bf16 && d == kSegD && chunk == 16 && T >= 2048 && BH >= 1 &&
           (long)BH * 4 <= kSegUnits && (long long)T * d * 2 < 0x7fffffffLL &&
           (long long)BH * T * d * 2 <= 0x7fffffffffffLL;
}

// Whether the plan beats the one-segment chain kernel.  Up to 32 slices (at least
// eight segments each) it does from T = 2048 on.  From 33 to 64 slices, five to
// eight segments: measured per call, 1 x 40 heads T = 4096 43.7 against 52.0 us,
// 1 x 48 heads T = 8192 70.0 against 98.8 us, 2 x 32 heads T = 32768 305.5
// against 410.0 us, but 2 x 32 heads T = 2048 36.7 against 29.0 us.
bool linear_seg_preferred(int BH, int T)
{
    return BH <= kSegUnits / 8 || T >= 4096;
}

size_t linear_seg_workspace(int BH, int T, int d)
{
    (void)d;
    const SegPlan p = seg_plan(BH, T);
    return 3 * (size_t)BH * p.S * kSegD * kSegD * sizeof(float);
}

hipError_t launch_linear_seg(const LinearArgs& a, hipStream_t s)
{
    if (!a.eta) return launch_seg_eta<kSegEtaScalar>(a, s);
    // 16-byte eta loads need every slice's rows 16-byte aligned
    if (reinterpret_cast<uintptr_t>(a.eta) % 16 == 0 && a.T % 4 == 0)
        return launch_seg_eta<kSegEtaToken4>(a, s);
    return launch_seg_eta<kSegEtaToken>(a, s);
}

}  // namespace ttt
