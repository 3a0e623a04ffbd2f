// TTT-Linear forward scan, chunks of exactly 16 tokens: each (batch, head) is
// split over d/16 / WPG workgroups of WPG waves, wave w of part p owning state
// rows 16 (p WPG + w) .. + 15.
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
// with the feature in the lanes for the state update).  V and eta are loaded per
// wave.  The parts of one head run on one XCD, so a tile fetched by one part is
// served to the other from that XCD's L2 (the HBM traffic stays one fetch per
// tile).
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

template <int D, int WPG, int ETA, bool FULL>
__global__ __launch_bounds__(64 * WPG) void linear_coop_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, int BH, int T)
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
    __shared__ KQTile16<D> L[kSlots];

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
    const size_t tok0 = (size_t)slice * T;
    const int nch = (T + 15) / 16;
    const int out0 = 16 * (part * WPG + wave);
    // token of row r of chunk ch, clamped into the sequence (a clamped row is a
    // re-read; its token gets eta = 0 and no store)
    auto tok = [&](int ch, int r) {
        const int cc = ch < nch ? ch : nch - 1;
        const int t = 16 * cc + r;
        return FULL ? t : (t < T ? t : T - 1);
    };

    // this thread's granules of each staged tile: granule tid + i NT of the 32 G
    // granules of K (the first 16 G) and Q
    int which[GPT], grow[GPT], ggr[GPT], lpos[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int idx = tid + i * NT;
        which[i] = idx / (16 * G);
        grow[i] = (idx / G) & 15;
        ggr[i] = idx % G;
        lpos[i] = grow[i] * G + (ggr[i] ^ tile16_swizzle<D>(grow[i]));
    }
    // first token of chunk ch (clamped), as a wave-uniform base; lanes add a
    // 32-bit offset within the chunk
    auto chunk_base = [&](int ch) {
        const int cc = ch < nch ? ch : nch - 1;
        return tok0 + (size_t)16 * cc;
    };
    auto row_in = [&](int ch, int r) {   // row r of chunk ch, clamped into the sequence
        if (FULL) return r;
        const int cc = ch < nch ? ch : nch - 1;
        return 16 * cc + r < T ? r : T - 1 - 16 * cc;
    };
    auto gload = [&](u32x4 (&r)[GPT], int ch) {
        const size_t base = chunk_base(ch) * D;
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            r[i] = *(const u32x4*)((which[i] ? Q : K) + base + (row_in(ch, grow[i]) * D + 8 * ggr[i]));
    };
    auto gstore = [&](KQTile16<D>& t, const u32x4 (&r)[GPT]) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) t.g[which[i]][lpos[i]] = r[i];
    };
    auto vload = [&](int ch) {
        const uint16_t* b = V + chunk_base(ch) * D;
        return *(const u32x2*)(b + (row_in(ch, c) * D + out0 + 4 * g));
    };
    auto eload = [&](int ch) {
        if (ETA == kCoopEtaToken4) {
            const int cc = ch < nch ? ch : nch - 1;
            return *(const f32x4*)(eta + tok0 + 16 * cc + 4 * g);
        } else if (ETA == kCoopEtaToken) {
            f32x4 e;
#pragma unroll
            for (int r = 0; r < 4; ++r) e[r] = eta[tok0 + tok(ch, 4 * g + r)];
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
    u32x4 Mf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
    const u32x2 I16 = identity_b16(lane);

    // chunk X lives in LDS slot X % kSlots.  Tiles of chunks 0 .. P-1 are
    // stored up front; during chunk ch the tile of chunk ch + P is stored and the
    // granule of chunk ch + 2P loaded (into the register slot it came from).
    u32x4 rg[P][GPT];
    u32x2 rv[P];
    f32x4 re[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        gload(rg[p], p);
        rv[p] = vload(p);
        re[p] = eload(p);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        gstore(L[p], rg[p]);
        gload(rg[p], P + p);
    }
    __syncthreads();

    // E_0 = K_0 W_0^T - V_0 directly.  kb[ch & 1] holds K_ch as row operand; the
    // other set holds K_{ch+1}.
    u32x4 kb[2][NM];
    row_operand(L[0].g[0], kb[0]);
    row_operand(L[1].g[0], kb[1]);
    f32x4 Et = mfma16(rv[0] ^ u32x2{0x80008000u, 0x80008000u}, I16, f32x4{0, 0, 0, 0});
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
        // stage chunk ch + P, refill its register slot with chunk ch + 2P
        if (ch + P < nch) gstore(L[(k + P) % kSlots], rg[p]);
        gload(rg[p], ch + 2 * P);

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
        f32x4 et = re[p];
        if (!FULL) {
            const int n = min(16, T - 16 * ch);
            et.x = (4 * g + 0 < n) ? et.x : 0.f;
            et.y = (4 * g + 1 < n) ? et.y : 0.f;
            et.z = (4 * g + 2 < n) ? et.z : 0.f;
            et.w = (4 * g + 3 < n) ? et.w : 0.f;
        }
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
            const u32x2 vneg = rv[(p + 1) % P] ^ u32x2{0x80008000u, 0x80008000u};
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
        if (FULL || 16 * ch + c < T) {
            uint16_t* zb = Z + (tok0 + (size_t)16 * ch) * D;
            *(u32x2*)(zb + (c * D + out0 + 4 * g)) = pack_bf16x4(Zt);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
        // K_{c+2} into the set K_c leaves (stale, unused, past the end)
        row_operand(L[(k + 2) % kSlots].g[0], kc);
        rv[p] = vload(ch + P);
        re[p] = eload(ch + P);
        if (p % kGroup == kGroup - 1) __syncthreads();
    };

    int c0 = 0;
    for (; c0 + kSlots <= nch; c0 += kSlots)
        unroll_seq([&](auto k) { step(c0 + k, k); }, std::make_integer_sequence<int, kSlots>{});
    unroll_seq([&](auto k) {
        if (c0 + k < nch) step(c0 + k, k);
    }, std::make_integer_sequence<int, kSlots - 1>{});

    float* w = W_out + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        *(f32x4*)(w + 32 * m + 8 * g) = M[2 * m];
        *(f32x4*)(w + 32 * m + 8 * g + 4) = M[2 * m + 1];
    }
}

template <int D, int WPG, int ETA, bool FULL>
void launch_cfg(const LinearArgs& a, hipStream_t s)
{
    constexpr int parts = D / 16 / WPG;
    const unsigned grid = parts == 1 ? (unsigned)a.BH : (unsigned)((a.BH + 7) / 8 * 8 * parts);
    hipLaunchKernelGGL((linear_coop_kernel<D, WPG, ETA, FULL>), dim3(grid), dim3(64 * WPG), 0,
                       s, (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta,
                       a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.BH, a.T);
}

template <int D, int WPG>
void launch_eta(const LinearArgs& a, hipStream_t s)
{
    const bool full = a.T % 16 == 0;
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
    switch (a.d) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ttt
