// TTT-Linear forward scan, chunks of exactly 16 tokens: each (batch, head) is
// split over d/16 / WPG workgroups of WPG waves, wave w of part p owning state
// rows 16 (p WPG + w) .. + 15.  Packed documents take the ragged-chunk form
// (FULL false) with one slice per (document, head): its tokens come from the
// offset table, and an empty document copies its start state through.
//
// Same chunk arithmetic as the single-wave chunk kernel (linear_mfma.hip): with
// F_c = -diag(eta) E_c (token-row layout, PaperTrace "5 · TestingTime 训练与长上下文"
// §1.1/§2.3, dual form of diosapp "Test-Time Training (TTT) guide" §3)
//     Z_c     = Q_c W_c^T + (causal, inclusive Q_c K_c^T) F_c,
//     W_{c+1} = W_c + F_c^T K_c,
//     E_{c+1} = [K_{c+1} W_c^T - V_{c+1}] + (K_{c+1} K_c^T) F_c   (Gram lookahead).
//
// Every wave of a head needs the whole K and Q tile of each chunk.  Instead of
// each wave fetching them (d/16 copies through the compute unit's vector-memory
// path, which saturates once several waves share a compute unit), the workgroup
// fetches each tile once -- one coalesced 16-byte granule per thread, through a
// register ring -- into a ring of swizzled LDS tiles (below), and
// every wave reads its operands from there (row reads; the transpose read gives K
// with the feature in the lanes for the state update).  The parts of one head run
// on one XCD, so a tile fetched by one part is served to the other from that
// XCD's L2 (the HBM traffic stays one fetch per tile).
//
// A compute unit's vector-memory path pays per cache line an instruction touches
// more than per byte, so with four waves at d = 64 V and Z also move as contiguous
// pieces: the workgroup's
// feature stripe of a chunk (16 tokens x 16 WPG features) is loaded as one 8-byte
// piece per thread into the LDS tile, and Z leaves through an LDS stage one group
// of chunks later, after the barrier that makes every wave's part visible, one
// 8-byte piece per thread (a range-checked buffer store drops rows past T).  Each
// wave reads its 16 x 16 block of V from LDS.  eta stays a per-lane load (the
// four tokens of the lane's rows).  Elsewhere each wave loads its V block and
// stores its Z block itself: at d = 128 the extra LDS and registers do not fit
// beside the K and Q rings, and two-wave workgroups at d = 64 (a 64-byte stripe
// per token) measured slower staged (8x12 heads, T = 2048: 37.5 us against 36.3;
// four-wave workgroups at 64x12 heads, T = 1024: 94.0 against 99.7).
//
// A sequence whose length is not a multiple of 16 (and every packed document)
// takes the ragged form: its loads and stores go through range-checked buffer
// resources over the slice's rows, so rows past the end read as zero and are not
// written, and a zero row of K and V contributes nothing to the scan.  The loop
// then has no per-lane clamps, masks or branches and runs at the whole-chunk rate
// (8x12 heads, T = 2047: 36.8 us, against 48.3 with clamped loads and masked eta;
// 8 packed documents of 8x12 heads' tokens: 58.6 against 78.0).
//
// Tiles are staged P = 2 kGroup chunks ahead into a ring of 2P LDS slots, with
// one barrier per kGroup chunks: a slot is rewritten only once every wave has
// passed the chunks that read it.  The loop is unrolled over the whole ring, so
// every slot address is a compile-time offset.  The K rows of chunk c+2 are read
// into registers during chunk c, keeping LDS latency off the chunk-to-chunk
// chain.
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace ttt {
namespace {

enum { kCoopEtaScalar = 0, kCoopEtaToken = 1, kCoopEtaToken4 = 2 };

// f(integral_constant<int, I>) for I = 0, 1, ... in order
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
constexpr long kComputeUnits = 256;   // MI355X

typedef __attribute__((ext_vector_type(2))) int i32x2;

// K and Q as swizzled 16-byte granules; V as 8-byte units (four features) of the
// workgroup's stripe, unit u of token r at r U + (u ^ coop_vswz(r)) with U = 4 WPG
// units per token: the 16 tokens a lane group reads at one unit fall on distinct
// banks.
template <int D, int WPG>
struct CoopTile {
    u32x4 g[2][16 * (D / 8)];
    u32x2 v[D == 64 && WPG >= 4 ? 16 * 4 * WPG : 1];
};

__device__ __forceinline__ int coop_vswz(int r) { return (r >> 1) & 7; }

constexpr int kCoopBufferFlags = 0x00020000;   // dword 3 of a gfx9 buffer resource: raw 32-bit data
// K, Q and V bytes are read once per workgroup and Z bytes written once, so they
// go with the non-temporal bit of gfx950's cache-policy operand (for pointer
// accesses, the nontemporal builtins).  The second workgroup of a split head still
// finds the K and Q tiles in L2.  eta keeps the default policy: every wave reads
// each of its lines.  8 x 12 heads, T = 2048: 36.9 -> 36.2 us per call.
constexpr int kCoopStream = 2;

template <int D, int WPG, int ETA, bool FULL>
__global__ __launch_bounds__(64 * WPG) void linear_coop_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, int BH, int T_all,
    const int* __restrict__ cu, int H, int total_T)
{
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    constexpr int G = D / 8;           // 16-byte granules per row
    constexpr int NT = 64 * WPG;       // threads per workgroup
    constexpr int GPT = 32 * G / NT;   // granules of a chunk's K and Q tiles per thread
    constexpr int PARTS = NB / WPG;    // workgroups per head
    static_assert(NB % WPG == 0 && GPT >= 1 && GPT * NT == 32 * G, "tile split");
    // chunks per barrier (eight waves per workgroup leave 256 registers per wave,
    // so shorter rings)
    constexpr int kGroup = WPG >= 8 ? 2 : 4;
    constexpr int P = 2 * kGroup;   // chunks whose granules a thread holds in registers
    constexpr int kSlots = 2 * P;   // > P + kGroup: chunks ch - kGroup .. ch + 2 stay
    constexpr bool SV = D == 64 && WPG >= 4;   // V staged through LDS
    constexpr bool SZ = D == 64 && WPG >= 4;   // Z staged through LDS
    constexpr int U = 4 * WPG;      // 8-byte units of the stripe per token
    __shared__ CoopTile<D, WPG> L[kSlots];
    __shared__ u32x2 Zs[SZ ? 2 * kGroup : 1][SZ ? 16 * U : 1];   // Z of two groups of chunks

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    int slice, part;
    if constexpr (PARTS == 1) {
        slice = blockIdx.x;
        part = 0;
    } else {
        xcd_unit_part(blockIdx.x, PARTS, slice, part);
        if (slice >= BH) return;
    }
    // the slice's first row and length T (packed documents: only with a ragged
    // last chunk, FULL false)
    size_t tok0;
    int T;
    if constexpr (FULL) {
        tok0 = (size_t)slice * T_all;
        T = T_all;
    } else {
        slice_span(cu, H, total_T, T_all, slice, tok0, T);
    }
    const int nch = (T + 15) / 16;
    const int out0 = 16 * (part * WPG + wave);
    // Ragged form: K, Q, V, eta and Z go through range-checked buffer resources
    // over the slice's rows, the whole offset in the vector offset (the part the
    // check covers; T d 2 < 2^31 - 2^20, so that offsets past the end still fit):
    // rows past T and chunks past the end read as zero, and Z rows past T are
    // dropped.  A zero row of K and V gives a zero row of E, so such a token
    // contributes nothing (F row zero) whatever its eta: no clamps, masks or
    // per-lane branches.
    auto rsrc = [](const void* base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kCoopBufferFlags);
    };
    const int sbytes = FULL ? 0 : T * D * 2;
    const auto bK = rsrc(K + tok0 * D, sbytes), bQ = rsrc(Q + tok0 * D, sbytes);
    const auto bV = rsrc(V + tok0 * D, sbytes), bZ = rsrc(Z + tok0 * D, sbytes);
    const auto bE = rsrc(eta ? eta + tok0 : nullptr, eta && !FULL ? T * 4 : 0);
    const int sbase = 16 * WPG * part;   // first feature of the workgroup's stripe
    // thread tid's piece of a stripe tile: token vrow, unit vunit; this lane's
    // unit of one (token c, features out0 + 4g .. + 3)
    const int vrow = tid / U, vunit = tid % U;
    const int vpos = vrow * U + (vunit ^ coop_vswz(vrow));
    const int opos = c * U + ((4 * wave + g) ^ coop_vswz(c));

    // this thread's granules of each staged tile: granule tid + i NT of the 32 G
    // granules of K (the first 16 G) and Q
    // (a wave's granules all come from one of the two: which[i] is also
    // (64 wave + i NT) / 16 G, uniform)
    static_assert(16 * G % 64 == 0, "a wave's granules lie in one tile");
    int which[GPT], grow[GPT], ggr[GPT], lpos[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int idx = tid + i * NT;
        which[i] = idx / (16 * G);
        grow[i] = (idx / G) & 15;
        ggr[i] = idx % G;
        lpos[i] = grow[i] * G + (ggr[i] ^ tile16_swizzle<D>(grow[i]));
    }
    // whole-chunk form: first token of chunk ch (a chunk past the end re-reads the
    // last one), as a wave-uniform base; lanes add a 32-bit offset within the chunk
    auto chunk_base = [&](int ch) {
        const int cc = ch < nch ? ch : nch - 1;
        return tok0 + (size_t)16 * cc;
    };
    auto gload = [&](u32x4 (&r)[GPT], int ch) {
        if constexpr (FULL) {
            const size_t base = chunk_base(ch) * D;
#pragma unroll
            for (int i = 0; i < GPT; ++i)
                r[i] = __builtin_nontemporal_load(
                    (const u32x4*)((which[i] ? Q : K) + base + (grow[i] * D + 8 * ggr[i])));
        } else {
#pragma unroll
            for (int i = 0; i < GPT; ++i)
                r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    (64 * wave + i * NT) / (16 * G) ? bQ : bK,
                    (16 * ch + grow[i]) * (2 * D) + 16 * ggr[i], 0, kCoopStream));
        }
    };
    auto stage = [&](CoopTile<D, WPG>& t, const u32x4 (&r)[GPT], const u32x2& v) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) t.g[which[i]][lpos[i]] = r[i];
        if constexpr (SV) t.v[vpos] = v;
    };
    // SV: thread tid's piece of the stripe; else this lane's unit
    auto vload = [&](int ch) {
        const int r = SV ? vrow : c, f = SV ? sbase + 4 * vunit : out0 + 4 * g;
        if constexpr (FULL) {
            return __builtin_nontemporal_load((const u32x2*)(V + chunk_base(ch) * D + (r * D + f)));
        } else {
            return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                bV, ((16 * ch + r) * D + f) * 2, 0, kCoopStream));
        }
    };
    // Z of chunk ch as thread tid's piece: rows past T (and chunks ch < 0) fall
    // outside the resource and are dropped
    auto zstore = [&](const u32x2& v, int ch) {
        const int rows = ch < 0 ? 0 : min(16, T - 16 * ch);
        const auto rz = __builtin_amdgcn_make_buffer_rsrc(
            Z + (tok0 + (size_t)16 * (ch < 0 ? 0 : ch)) * D, 0, rows * D * 2, kCoopBufferFlags);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), rz,
                                              (vrow * D + sbase + 4 * vunit) * 2, 0, kCoopStream);
    };
    auto eload = [&](int ch) {
        if (ETA == kCoopEtaToken4) {
            const int cc = ch < nch ? ch : nch - 1;
            return *(const f32x4*)(eta + tok0 + 16 * cc + 4 * g);
        } else if (ETA == kCoopEtaToken) {
            f32x4 e;
            if constexpr (FULL) {
                const int cc = ch < nch ? ch : nch - 1;
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = eta[tok0 + 16 * cc + 4 * g + r];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    e[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        bE, (16 * ch + 4 * g + r) * 4, 0, 0));
            }
            return e;
        } else {
            return f32x4{eta_scalar, eta_scalar, eta_scalar, eta_scalar};
        }
    };
    // row operand of a staged tile: lane (c, g) gets granules 4m + g of row c
    auto row_operand = [&](const u32x4* t, u32x4 (&op)[NM]) {
#pragma unroll
        for (int m = 0; m < NM; ++m) op[m] = t[c * G + ((4 * m + g) ^ tile16_swizzle<D>(c))];
    };

    f32x4 M[NB];
    {
        const float* w = W0 + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[2 * m] = *(const f32x4*)(w + 32 * m + 8 * g);
            M[2 * m + 1] = *(const f32x4*)(w + 32 * m + 8 * g + 4);
        }
    }
    // this wave's rows of the state to W_out
    auto store_state = [&]() {
        float* w = W_out + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            *(f32x4*)(w + 32 * m + 8 * g) = M[2 * m];
            *(f32x4*)(w + 32 * m + 8 * g + 4) = M[2 * m + 1];
        }
    };
    if (!FULL && T == 0) {   // an empty document (uniform over the workgroup): the state passes through
        store_state();
        return;
    }
    u32x4 Mf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
    const u32x2 I16 = identity_b16(lane);

    // chunk X lives in LDS slot X % kSlots.  Tiles of chunks 0 .. P-1 are
    // stored up front; during chunk ch the tile of chunk ch + P is stored and the
    // pieces of chunk ch + 2P loaded (into the register slots they came from).
    // re[] holds eta of chunks ch .. ch + P - 1, and so does rv[] when V is not
    // staged.
    u32x4 rg[P][GPT];
    u32x2 rv[P];
    f32x4 re[P];
    if constexpr (SV) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            gload(rg[p], p);
            rv[p] = vload(p);
        }
        // the loads that stay in flight into the loop, in the order a chunk step
        // issues them, so that the loop's waits count them as in the steady state
#pragma unroll
        for (int p = 0; p < P; ++p) {
            stage(L[p], rg[p], rv[p]);
            gload(rg[p], P + p);
            rv[p] = vload(P + p);
            re[p] = eload(p);
        }
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            gload(rg[p], p);
            rv[p] = vload(p);
            re[p] = eload(p);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            stage(L[p], rg[p], rv[p]);
            gload(rg[p], P + p);
        }
    }
    __syncthreads();
    // -V of chunk ch + 1 for the lookahead, ch at ring position k
    auto vneg_next = [&](auto kc_) {
        constexpr int k = decltype(kc_)::value;
        if constexpr (SV) return L[(k + 1) % kSlots].v[opos] ^ u32x2{0x80008000u, 0x80008000u};
        else return rv[(k % P + 1) % P] ^ u32x2{0x80008000u, 0x80008000u};
    };

    // E_0 = K_0 W_0^T - V_0 directly.  kb[ch & 1] holds K_ch as row operand; the
    // other set holds K_{ch+1}.
    u32x4 kb[2][NM];
    row_operand(L[0].g[0], kb[0]);
    row_operand(L[1].g[0], kb[1]);
    const u32x2 v0 = SV ? L[0].v[opos] : rv[0];
    f32x4 Et = mfma16(v0 ^ u32x2{0x80008000u, 0x80008000u}, I16, f32x4{0, 0, 0, 0});
#pragma unroll
    for (int m = 0; m < NM; ++m) Et = mfma32(kb[0][m], Mf[m], Et);

    // 16-deep products as 32-deep ones whose lower half is zero in one operand
    // (the other holds the identity there): these tuples live across the loop,
    // their lower halves never written, so no zeros are moved in per product
    u32x4 ktz[NB], smz = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) ktz[jb] = u32x4{0u, 0u, 0u, 0u};

    // one chunk; k = ch % kSlots is a compile-time ring position
    auto step = [&](int ch, auto kc_) {
        constexpr int k = decltype(kc_)::value;
        constexpr int p = k % P;
        constexpr int j = k % kGroup;              // chunk within its group
        constexpr int zb = (k / kGroup) & 1;       // group parity (kSlots is a multiple of 2 kGroup)
        // stage chunk ch + P, refill its register slots with chunk ch + 2P.  With V
        // staged this is unconditional: past the end the slot receives a re-read of
        // the last chunk (read only by the unused lookahead), and a conditional use
        // would let the compiler sink the prefetch loads into the branch.
        // Otherwise the conditional form, which keeps d = 128 under the register
        // limit.
        if (SV || ch + P < nch) stage(L[(k + P) % kSlots], rg[p], rv[p]);
        gload(rg[p], ch + 2 * P);
        if constexpr (SV) rv[p] = vload(ch + 2 * P);
        // the previous group's Z, complete since the last barrier
        u32x2 zprev = {0u, 0u};
        if constexpr (SZ) zprev = Zs[(zb ^ 1) * kGroup + j][vpos];

        constexpr int sl = k;
        const u32x4* Kc = L[sl].g[0];
        const u32x4* Qc = L[sl].g[1];
        constexpr int pe = p & 1;   // ch & 1 (the ring length is even)
        u32x4 (&kc)[NM] = kb[pe];
        u32x4 (&kn)[NM] = kb[pe ^ 1];
        u32x4 qc[NM];
        row_operand(Qc, qc);
        // K_c with the feature in the lanes (A operand of the state update), in
        // the upper half of the zero-padded operands
        {
            const int r = (lane >> 2) & 3, q = lane & 3;
            const int row = 4 * g + r;
            const u32x2* base = reinterpret_cast<const u32x2*>(Kc) + row * (2 * G);
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                auto pt = (__attribute__((address_space(3))) s16x4*)(
                    base + 2 * ((4 * (jb >> 1) + q) ^ tile16_swizzle<D>(row)) + (jb & 1));
                const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(pt));
                ktz[jb].z = t.x;
                ktz[jb].w = t.y;
            }
        }
        const f32x4 et = re[p];
        // F_c = -diag(eta) E_c: the only value the next chunk waits for
        const u32x2 F = pack_bf16x4(-et * Et);
        const u32x4 IF = {I16.x, I16.y, F.x, F.y};
        // E_{c+1} = K_{c+1} W_c^T + [-V_{c+1} | G_c] [I ; F_c]
        {
            f32x4 Gt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Gt = mfma32(kc[m], kn[m], Gt);
            const u32x2 Gb = pack_bf16x4(Gt);
            f32x4 Pt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Pt = mfma32(kn[m], Mf[m], Pt);
            const u32x2 vneg = vneg_next(kc_);
            Et = mfma32(u32x4{vneg.x, vneg.y, Gb.x, Gb.y}, IF, Pt);
        }
        // W_{c+1} = W_c + F_c^T K_c: [0 | K_c^T] [I ; F_c]
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) M[jb] = mfma32(ktz[jb], IF, M[jb]);
        // Z_c = Q_c W_c^T + causal scores times F_c
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
        {   // + [I | F_c^T] [0 ; causal scores]
            const u32x2 sb = pack_bf16x4(Sm);
            smz.z = sb.x;
            smz.w = sb.y;
            Zt = mfma32(IF, smz, Zt);
        }
        if constexpr (SZ) {
            Zs[zb * kGroup + j][opos] = pack_bf16x4(Zt);
            zstore(zprev, ch - kGroup);
        } else if constexpr (FULL) {
            uint16_t* zp = Z + (tok0 + (size_t)16 * ch) * D;
            __builtin_nontemporal_store(pack_bf16x4(Zt), (u32x2*)(zp + (c * D + out0 + 4 * g)));
        } else {
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, pack_bf16x4(Zt)), bZ,
                                                  ((16 * ch + c) * D + out0 + 4 * g) * 2, 0,
                                                  kCoopStream);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
        // K_{c+2} into the set K_c leaves (stale, unused, past the end)
        row_operand(L[(k + 2) % kSlots].g[0], kc);
        if constexpr (!SV) rv[p] = vload(ch + P);
        re[p] = eload(ch + P);
        if (j == kGroup - 1) __syncthreads();
    };

    int c0 = 0;
    for (; c0 + kSlots <= nch; c0 += kSlots)
        unroll_seq([&](auto k) { step(c0 + k, k); }, std::make_integer_sequence<int, kSlots>{});
    unroll_seq([&](auto k) {
        if (c0 + k < nch) step(c0 + k, k);
    }, std::make_integer_sequence<int, kSlots - 1>{});

    if constexpr (SZ) {   // Z of the last group and the rest of the group before it
        __syncthreads();
        const int gl = (nch - 1) / kGroup, m = nch - gl * kGroup;
        if (gl > 0)
            for (int jj = m; jj < kGroup; ++jj)
                zstore(Zs[((gl - 1) & 1) * kGroup + jj][vpos], (gl - 1) * kGroup + jj);
        for (int jj = 0; jj < m; ++jj) zstore(Zs[(gl & 1) * kGroup + jj][vpos], gl * kGroup + jj);
    }

    store_state();
}

template <int D, int WPG, int ETA, bool FULL>
void launch_cfg(const LinearArgs& a, hipStream_t s)
{
    constexpr int parts = D / 16 / WPG;
    const unsigned grid = parts == 1 ? (unsigned)a.BH : (unsigned)((a.BH + 7) / 8 * 8 * parts);
    hipLaunchKernelGGL((linear_coop_kernel<D, WPG, ETA, FULL>), dim3(grid), dim3(64 * WPG), 0,
                       s, (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta,
                       a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.BH, a.T, a.cu, a.H,
                       a.total_T);
}

template <int D, int WPG>
void launch_eta(const LinearArgs& a, hipStream_t s)
{
    const bool full = !a.cu && a.T % 16 == 0;
    const bool eta4 = a.eta && full && reinterpret_cast<uintptr_t>(a.eta) % 16 == 0;
    if (full) {
        if (!a.eta) launch_cfg<D, WPG, kCoopEtaScalar, true>(a, s);
        else if (eta4) launch_cfg<D, WPG, kCoopEtaToken4, true>(a, s);
        else launch_cfg<D, WPG, kCoopEtaToken, true>(a, s);
    } else {
        if (!a.eta) launch_cfg<D, WPG, kCoopEtaScalar, false>(a, s);
        else launch_cfg<D, WPG, kCoopEtaToken, false>(a, s);
    }
}

// Waves per workgroup, measured on MI355X at T = 2048: a head is split over
// workgroups while they find a compute unit each.  d = 64: two workgroups of two
// waves (8x12 heads: 39.0 us against 48.9 with one of four; 8x12 heads at
// T = 8192: 130 against 173 us).  d = 128: two workgroups of four waves (4x12
// heads: 71.8 us against 106.4 with eight waves; 8x12: 84.8 against 113.2); two
// waves measured no faster there (4x12: 74.0 us).
template <int D>
hipError_t launch_d(const LinearArgs& a, hipStream_t s)
{
    if (a.BH * 2 > kComputeUnits) launch_eta<D, D / 16>(a, s);
    else launch_eta<D, D == 64 ? 2 : 4>(a, s);
    return hipGetLastError();
}

}  // namespace

bool linear_coop_supported(int d, int chunk, int bf16)
{
    return bf16 && (d == 64 || d == 128) && chunk == 16;
}

hipError_t launch_linear_coop(const LinearArgs& a, hipStream_t s)
{
    // the ragged form (packed documents, or T not a multiple of 16) addresses a
    // slice through 32-bit buffer offsets
    const long long span = a.cu ? a.total_T : a.T;
    if (!(!a.cu && a.T % 16 == 0) && span * a.d * 2 >= (1LL << 31) - (1LL << 20))
        return hipErrorInvalidValue;
    switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ttt
