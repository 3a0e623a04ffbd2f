// Backward pass (vector-Jacobian product) of the TTT-Linear scan.
//
// Forward, per chunk of b tokens with chunk-start state W (PaperTrace "5 ·
// TestingTime 训练与长上下文" §1.1, §2.1, §2.3): E = W K - V, F = E diag(eta),
// Z = W Q - F (U o K^T Q), W_next = W - F K^T, with tokens as columns and U the
// causal mask (s <= t).  Given the cotangents dZ and dW_next, the chunk's
// gradients are, in 16-token sub-tiles sigma taken from the last
// (P = dW_next + sum over later sub-tiles of dZ_tau Q_tau^T,
//  H = W - G_{<sigma}, G_{<sigma} the chunk's update before sub-tile sigma):
//   dF    = -dZ (U o K^T Q)^T - P K          (only the diagonal sub-tile masked)
//   dE    = dF diag(eta),  deta_s = e_s . dF_s,  dV = -dE
//   dA    = -(F^T dZ) o U
//   dK    = -P^T F + Q dA^T + W^T dE          (tokens x dims: -F^T P + dA Q + dE^T W)
//   dQ    = H^T dZ + K dA
//   dW    = P_final + sum_sigma dE K^T        (= the previous chunk's dW_next)
// Every product above except the sums behind dK, dQ and deta is separable by
// state row: a workgroup owns 16 rows of one (batch, head) state, runs the
// forward recurrence for them (saving each chunk-start state to the workspace),
// then the reverse recurrence.  Its waves split the state's column blocks: each
// keeps its blocks of W, P, dW and H and computes its blocks of dK and dQ, and
// the contractions over all columns (E, P K^T, K Q^T) are summed from per-wave
// partial tiles in LDS.  Contributions to dK, dQ and deta (sums over the rows)
// go to one fp32 plane per row block, each element written once; a last pass
// adds the planes in row-block order (and rounds to bf16 with bf16 I/O), so the
// results are the same bits on every call.
//
// With chunks of at most 16 tokens and fewer units than compute units, each
// sequence is also cut into segments along T, one unit per (sequence, row block,
// segment): the unit recomputes the forward up to its segment's end, carries the
// state's cotangent back from dW_T over the later segments (the affine reverse
// recurrence, from K, Q, dZ and eta only) and runs the full reverse over its own
// segment, with the bits of the one-segment pass.
//
// Every product is a 16 x 16 tile product, operands staged through LDS in
// row-major fp32 tiles with padded rows.  With fp32 I/O it runs on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32); with bf16 I/O on the bf16 ones, the
// fp32 operands of the reverse recurrence split as hi + lo bf16 (mmt in
// mfma_f32.h: about 2^-17 relative per product) and those of the dK and dQ
// products rounded to bf16, the outputs' own precision.  Register forms
// of a 16 x 16 tile X (lane l, c = l % 16, g = l / 16, slot v = 0..3):
//   CL(X): lane holds X[4g + v][c]   (the MFMA result layout; a B operand whose
//                                     contraction index is X's row)
//   RL(X): lane holds X[c][4g + v]   (an A operand whose contraction index is
//                                     X's column)
// and RL(X) = CL(X^T).
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"
#include "mfma_f32.h"

namespace ttt {

namespace {

typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kSub = 16;   // tokens per sub-tile

// A1 B1 + A2 B2 + C for two 16 x 16 tile products (RL / CL operands): with bf16
// operands one 16x16x32 instruction holds both, the first product in slots 0-3
// of each lane group and the second in slots 4-7 (operands rounded to bf16);
// otherwise two fp32 products
template <bool BF>
__device__ __forceinline__ f32x4 mm2(f32x4 a1, f32x4 b1, f32x4 a2, f32x4 b2, f32x4 acc)
{
    if constexpr (!BF) {
        return mm16(a2, b2, mm16(a1, b1, acc));
    } else {
        const u32x2 x1 = pack_bf16x4(a1), x2 = pack_bf16x4(a2);
        const u32x2 y1 = pack_bf16x4(b1), y2 = pack_bf16x4(b2);
        return mfma32(u32x4{x1.x, x1.y, x2.x, x2.y}, u32x4{y1.x, y1.y, y2.x, y2.y}, acc);
    }
}

// ---------------------------------------------------------------- global I/O
// Range-checked buffer accesses: a store or atomic add whose byte offset lies at
// or past the resource's size is dropped by the memory unit.  Lanes outside a
// sub-tile (or waves that must not write) point past the range instead of
// branching, so every wave issues the same memory operations and a later wait
// for prefetched loads need not cover them.
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a gfx9 buffer resource: raw 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                            kBufferFlags);
}

// four consecutive values of the I/O type at byte offset `off`
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v,
                                              float)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 0);
}

__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v,
                                              uint16_t)
{
    // hardware convert (round to nearest even): no branch for the NaN case
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, pack_bf16x4(v)), r, off, 0, 0);
}

// N consecutive elements (N a multiple of 4) widened to fp32
template <int N>
__device__ __forceinline__ void load_vec(const float* p, float* out)
{
#pragma unroll
    for (int i = 0; i < N; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + i);
        out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
    }
}

template <int N>
__device__ __forceinline__ void load_vec(const uint16_t* p, float* out)
{
#pragma unroll
    for (int i = 0; i < N; i += 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p + i);
        out[i] = __uint_as_float(v.x << 16);
        out[i + 1] = __uint_as_float(v.x & 0xffff0000u);
        out[i + 2] = __uint_as_float(v.y << 16);
        out[i + 3] = __uint_as_float(v.y & 0xffff0000u);
    }
}

// Waves per workgroup: each owns NB / NW of the d/16 column blocks.  With few
// (sequence, 16-row block) units the waves split a unit's work across SIMDs;
// once the units fill the compute units, one wave per unit (bf16 products, at
// d = 64) avoids the cross-wave sums and barriers.  Measured on MI355X with bf16
// I/O at d = 64: 8x12 heads (384 units) 0.598 -> 0.563 ms with one wave instead
// of four; 1x32 heads (128 units) 6.44 ms with four, 7.32 with one, 5.59 with two.
template <int D>
constexpr int bwd_waves()
{
    return D == 128 ? 2 : (D >= 32 ? D / 16 : 1);
}
constexpr long kComputeUnits = 256;
constexpr int kMaxBwdSeg = 8;

template <int D, int NW>
struct BwdLds {
    static constexpr int S = D + 4;   // row stride of the d-wide tiles
    float K[kSub * S];                // sub-tile keys    [token][dim]
    float Q[kSub * S];                // sub-tile queries [token][dim]
    float W[kSub * S];                // chunk-start state rows [row][dim] (own blocks per wave)
    float P[kSub * S];                // P rows [row][dim] (own blocks per wave)
    float V[kSub * 20];               // V of the block's dims  [token][row]
    float dZ[kSub * 20];              // dZ of the block's dims [token][row]
    float part[NW][3][kSub * 20];     // per-wave partial E, P K^T, K Q^T
    float M[NW][kSub * 20];           // masked K^T Q           [s][t]
    float dA[NW][kSub * 20];          // dA                     [s][t]
    float dE[NW][kSub * 20];          // dE                     [row][token]
    float F[NW][kSub * 20];           // F                      [row][token]
};

struct BwdArgs {
    const void* K;
    const void* Q;
    const void* V;
    const float* eta;
    float eta_scalar;
    const float* W0;
    const void* dZ;
    const float* dWT;     // may be null (zero)
    void* dV;
    float* dW0;
    float* states;        // [BH, nch + 1, d, d]
    float* dK_part;       // [d/16, BH, T, d] fp32: this row block's terms of dK
    float* dQ_part;       // [d/16, BH, T, d] fp32
    float* deta_part;     // [d/16, BH, T] fp32; null when deta is not wanted
    size_t plane;         // BH T d: elements of one dK / dQ plane
    size_t tplane;        // BH T: elements of one deta plane
    int BH, T, chunk;
    // segments along T (chunks of at most one sub-tile only): segment k owns
    // sub-tiles bound[k] .. bound[k + 1] - 1
    int nseg;
    int bound[kMaxBwdSeg + 1];
};

// N consecutive elements (N = 1, 2 or 4) widened to fp32
template <int N, typename TIO>
__device__ __forceinline__ void load_small(const TIO* p, float* out)
{
    if constexpr (N == 4) {
        load_vec<4>(p, out);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = io<TIO>::load(p, i);
    }
}

// One sub-tile's inputs, loaded into registers one sub-tile ahead.  The 64*NW
// threads share the K, Q (KP elements each) and V, dZ (VP elements each) tiles:
// thread t takes row t / (4 NW); every lane holds eta of token l % 16, and each
// wave the rows of its own column blocks of the chunk-start state (4 floats of
// row l / 4 per block) when the sub-tile opens a chunk in the reverse pass.
template <typename TIO, int D, int NW>
struct SubTile {
    static constexpr int KP = D / (4 * NW), VP = 4 / NW, NBW = D / 16 / NW;
    RawRow<TIO, KP> k, q;
    RawRow<TIO, VP> v, dz;
    RawRow<float, 4> w[NBW];
    float h[NBW][4];   // CL tiles of the state after the chunk (chunks of several sub-tiles)
    float eta;
    bool row_ok, eta_ok;   // rows and tokens past the sub-tile stage as zeros
};

// Element i of a raw row with its storage word ANDed with m (all ones or zero):
// zero bits widen to +0.0 in either I/O type.
template <typename TIO, int N>
__device__ __forceinline__ float masked_at(const RawRow<TIO, N>& r, int i, uint32_t m)
{
    if constexpr (sizeof(TIO) == 4) {
        return __uint_as_float(r.w[i] & m);
    } else {
        const uint32_t x = r.w[i >> 1] & m;
        return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
    }
}

// MULTI: chunks span several 16-token sub-tiles (the running W - G_{<sigma} is
// needed); a compile-time choice, so that chunks of at most 16 tokens carry no
// trace of it.
// SEG: segments along T (a.nseg > 1; MULTI false), a compile-time choice so that
// the one-segment pass carries no trace of them.
template <typename TIO, int D, int NW, bool MULTI, bool SEG = false>
__global__ __launch_bounds__(64 * NW) void linear_bwd_kernel(BwdArgs a)
{
    constexpr int NB = D / 16, NBW = NB / NW, S = D + 4;
    // bf16 I/O: K, Q, V and dZ values are exact in bf16 and the products run on
    // the bf16 matrix cores.  Products on the reverse recurrence (E, P K^T, the
    // scores, dF, dW, H) split their fp32 operands as hi + lo (about 17 bits);
    // those that only form the bf16 outputs dK and dQ (and dA, used only there)
    // round their operands to bf16, the outputs' own precision.  fp32 I/O keeps
    // fp32 products throughout.
    constexpr bool BF = sizeof(TIO) == 2;
    constexpr int KP = SubTile<TIO, D, NW>::KP, VP = SubTile<TIO, D, NW>::VP;
    __shared__ BwdLds<D, NW> L;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int srow = tid / (4 * NW), kcol = (tid % (4 * NW)) * KP, vcol = (tid % (4 * NW)) * VP;
    const int wrow = lane >> 2, wcol = (lane & 3) * 4;
    static_assert(!(SEG && MULTI), "segments take chunks of one sub-tile");
    int slice, part;
    xcd_unit_part(blockIdx.x, SEG ? NB * a.nseg : NB, slice, part);
    if (slice >= a.BH) return;
    const int rb = part % NB, seg = part / NB;
    const int r0 = 16 * rb;
    const int T = a.T, chunk = a.chunk;
    const int nch = (T + chunk - 1) / chunk;
    const int nsub = (chunk + kSub - 1) / kSub;            // sub-tiles of a full chunk
    const int last = (T - 1) / chunk * nsub + ((T - 1) % chunk) / kSub;   // last sub-tile
    // this unit's segment: sub-tiles j_lo .. j_hi (the whole sequence when nseg = 1)
    int j_lo = 0, j_hi = last;
    if constexpr (SEG) {
#pragma unroll
        for (int k = 0; k < kMaxBwdSeg; ++k) {
            if (k == seg) {
                j_lo = a.bound[k];
                j_hi = a.bound[k + 1] - 1;
            }
        }
    }
    const TIO* Kg = static_cast<const TIO*>(a.K) + (size_t)slice * T * D;
    const TIO* Qg = static_cast<const TIO*>(a.Q) + (size_t)slice * T * D;
    const TIO* Vg = static_cast<const TIO*>(a.V) + (size_t)slice * T * D;
    const TIO* dZg = static_cast<const TIO*>(a.dZ) + (size_t)slice * T * D;
    const float* etag = a.eta ? a.eta + (size_t)slice * T : nullptr;
    float* states = a.states + (size_t)slice * (nch + 1) * D * D;
    const size_t tokb = (size_t)slice * T;   // the slice's first token
    auto blk = [&](int bb) { return wave + NW * bb; };   // column block of slot bb

    // sub-tile j: chunk j / nsub, tokens [t0, t0 + len)
    auto span = [&](int j, int& ch, int& si, int& t0, int& len) {
        ch = j / nsub;
        si = j - ch * nsub;
        t0 = ch * chunk + si * kSub;
        len = min(kSub, min(ch * chunk + chunk, T) - t0);
    };
    auto fetch = [&](SubTile<TIO, D, NW>& f, int j, bool rev, bool state) {
        int ch, si, t0, len;
        span(j, ch, si, t0, len);
        // every load reads a row of the sub-tile (rows past its end re-read the
        // last one), so no register is written on a divergent path
        const size_t row = (size_t)(t0 + min(srow, len - 1)) * D;
        f.row_ok = srow < len;
        f.k.load(Kg + row + kcol);
        f.v.load(Vg + row + r0 + vcol);
        if (rev) {
            f.q.load(Qg + row + kcol);
            f.dz.load(dZg + row + r0 + vcol);
        }
        f.eta_ok = c < len;
        f.eta = etag ? etag[t0 + min(c, len - 1)] : a.eta_scalar;
        if (state) {
            const float* src = states + (size_t)ch * D * D + (size_t)(r0 + wrow) * D + wcol;
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb) f.w[bb].load(src + 16 * blk(bb));
            if constexpr (MULTI) {
                const float* hs = states + (size_t)(ch + 1) * D * D + (size_t)r0 * D;
#pragma unroll
                for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) f.h[bb][v] = hs[(4 * g + v) * D + 16 * blk(bb) + c];
            }
        }
    };
    auto put = [&](const SubTile<TIO, D, NW>& f, bool rev, bool state) {
        // Rows past the sub-tile stage as zeros through a mask on the raw words:
        // not a product (a re-read row may hold infinities) and not a select on
        // the values (that is compiled into a branch around the stores).
        const uint32_t m = f.row_ok ? 0xffffffffu : 0u;
        auto four = [&](const auto& r, int i) {
            return f32x4{masked_at(r, i, m), masked_at(r, i + 1, m), masked_at(r, i + 2, m),
                         masked_at(r, i + 3, m)};
        };
#pragma unroll
        for (int i = 0; i < KP; i += 4)
            *reinterpret_cast<f32x4*>(L.K + srow * S + kcol + i) = four(f.k, i);
#pragma unroll
        for (int i = 0; i < VP; ++i) L.V[srow * 20 + vcol + i] = masked_at(f.v, i, m);
        if (rev) {
#pragma unroll
            for (int i = 0; i < KP; i += 4)
                *reinterpret_cast<f32x4*>(L.Q + srow * S + kcol + i) = four(f.q, i);
#pragma unroll
            for (int i = 0; i < VP; ++i) L.dZ[srow * 20 + vcol + i] = masked_at(f.dz, i, m);
        }
        if (state) {
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb)
                *reinterpret_cast<f32x4*>(L.W + wrow * S + 16 * blk(bb) + wcol) =
                    f32x4{f.w[bb].at(0), f.w[bb].at(1), f.w[bb].at(2), f.w[bb].at(3)};
        }
    };
    auto store_state = [&](int slot, const f32x4* Wr) {
        float* dst = states + (size_t)slot * D * D + (size_t)r0 * D;
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
            for (int v = 0; v < 4; ++v) dst[(4 * g + v) * D + 16 * blk(bb) + c] = Wr[bb][v];
    };
    // sum of the waves' partial tiles k (same order in every wave: identical sums)
    auto reduce = [&](int k) {
        f32x4 r = cl<20>(L.part[0][k], 0, lane);
#pragma unroll
        for (int w = 1; w < NW; ++w) r += cl<20>(L.part[w][k], 0, lane);
        return r;
    };

    // two prefetch slots used alternately at compile-time positions: nothing is
    // copied out of registers that loads may still be filling
    SubTile<TIO, D, NW> bufs[2];

    // ------------------------------------------------ forward: chunk-start states
    f32x4 Wr[NBW];   // CL(W) of this wave's column blocks
#pragma unroll
    for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            Wr[bb][v] = a.W0[((size_t)slice * D + r0 + 4 * g + v) * D + 16 * blk(bb) + c];
    auto fwd_step = [&](int j, auto slot) {
        auto& cur = bufs[decltype(slot)::value];
        auto& nxt = bufs[decltype(slot)::value ^ 1];
        int ch, si, t0, len;
        span(j, ch, si, t0, len);
        __syncthreads();   // the previous sub-tile's tiles are consumed
        put(cur, false, false);
        // (after the staging, whose wait for the prefetched loads must not
        // cover these stores)
        if (si == 0) {
            if (j >= j_lo) store_state(ch, Wr);   // the segment's own chunk-start states
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb) put_cl<S>(L.W, 16 * blk(bb), lane, Wr[bb]);
        }
        const float et = cur.eta_ok ? cur.eta : 0.f;
        __syncthreads();
        if (j < j_hi) fetch(nxt, j + 1, false, false);
        // E = W K^T - V: this wave's part of the contraction over the state columns
        f32x4 Ew = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb)
            Ew = mmt<BF, false, true>(rl<S>(L.W, 16 * blk(bb), lane), rl<S>(L.K, 16 * blk(bb), lane), Ew);
        put_cl<20>(L.part[wave][0], 0, lane, Ew);
        __syncthreads();
        const f32x4 E = reduce(0);
        const f32x4 Vr = rl<20>(L.V, 0, lane);   // V[token c][row 4g + v], as E
        f32x4 Fm;   // -F
#pragma unroll
        for (int v = 0; v < 4; ++v) Fm[v] = -(E[v] - Vr[v]) * et;
        put_cl<20>(L.F[wave], 0, lane, Fm);
        lds_order();
        // W -= F K (contraction over the sub-tile's tokens), this wave's blocks
        const f32x4 Fa = rl<20>(L.F[wave], 0, lane);
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb)
            Wr[bb] = mmt<BF, false, true>(Fa, cl<S>(L.K, 16 * blk(bb), lane), Wr[bb]);
    };
    const std::integral_constant<int, 0> slot0;
    const std::integral_constant<int, 1> slot1;
    fetch(bufs[0], 0, false, false);
    {
        int j = 0;
        for (; j + 1 <= j_hi; j += 2) {
            fwd_step(j, slot0);
            fwd_step(j + 1, slot1);
        }
        if (j == j_hi) fwd_step(j, slot0);
    }
    if constexpr (MULTI) store_state(nch, Wr);
    __threadfence();   // the states are read back below
    __syncthreads();

    // ------------------------------------------------ reverse
    f32x4 P[NBW], dWa[NBW], Hr[NBW];
#pragma unroll
    for (int bb = 0; bb < NBW; ++bb) {
        dWa[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v)
            P[bb][v] = a.dWT ? a.dWT[((size_t)slice * D + r0 + 4 * g + v) * D + 16 * blk(bb) + c]
                             : 0.f;
    }
    // a sub-tile opens its chunk in the reverse pass when it is the chunk's last
    auto opens = [&](int j) {
        int ch, si, t0, len;
        span(j, ch, si, t0, len);
        return j == last || si == nsub - 1;
    };
    auto rev_step = [&](int j, auto slot) {
        auto& cur = bufs[decltype(slot)::value];
        auto& nxt = bufs[decltype(slot)::value ^ 1];
        int ch, si, t0, len;
        span(j, ch, si, t0, len);
        const bool first = opens(j);
        __syncthreads();   // the previous sub-tile's tiles are consumed
        put(cur, true, first);
        const float et = cur.eta_ok ? cur.eta : 0.f;
        if constexpr (MULTI) {
            if (first) {
#pragma unroll
                for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) Hr[bb][v] = cur.h[bb][v];
            }
        }
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) put_cl<S>(L.P, 16 * blk(bb), lane, P[bb]);
        __syncthreads();
        if (j > j_lo) fetch(nxt, j - 1, true, opens(j - 1));
        // partial E = W K^T, PK = P K^T, S = K Q^T over this wave's columns
        f32x4 Ew = {0.f, 0.f, 0.f, 0.f}, PKw = Ew, Sw = Ew;
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            const int b = blk(bb);
            const f32x4 kb = rl<S>(L.K, 16 * b, lane);
            Ew = mmt<BF, false, true>(rl<S>(L.W, 16 * b, lane), kb, Ew);
            PKw = mmt<BF, false, true>(rl<S>(L.P, 16 * b, lane), kb, PKw);
            Sw = mmt<BF, true, true>(kb, rl<S>(L.Q, 16 * b, lane), Sw);
        }
        put_cl<20>(L.part[wave][0], 0, lane, Ew);
        put_cl<20>(L.part[wave][1], 0, lane, PKw);
        put_cl<20>(L.part[wave][2], 0, lane, Sw);
        __syncthreads();
        f32x4 E = reduce(0);
        const f32x4 PK = reduce(1), Sm = reduce(2);
        const f32x4 Vr = rl<20>(L.V, 0, lane);
        f32x4 F, Mk;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            E[v] -= Vr[v];
            F[v] = E[v] * et;
            Mk[v] = (4 * g + v <= c) ? Sm[v] : 0.f;   // s = 4g + v, t = c
        }
        put_cl<20>(L.M[wave], 0, lane, Mk);
        lds_order();
        const f32x4 dZa = cl<20>(L.dZ, 0, lane);   // RL(dZ_blk): dZ[row c][token 4g + v]
        const f32x4 dZb = rl<20>(L.dZ, 0, lane);   // CL(dZ_blk): dZ[row 4g + v][token c]
        // dF = -dZ M^T - P K^T
        f32x4 dF = mmt<BF, true, false>(dZa, rl<20>(L.M[wave], 0, lane), f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 dE;
        float de = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            dF[v] = -dF[v] - PK[v];
            dE[v] = dF[v] * et;
            de += E[v] * dF[v];
        }
        // deta: sum over the block's 16 rows (4 slots x 4 lane groups); every wave
        // holds the same values, wave 0's are written (with dV); token c of the
        // sub-tile at byte 4c, dV row c at byte (c d + r0 + 4g) * size
        de += __shfl_xor(de, 16);
        de += __shfl_xor(de, 32);
        {
            const bool w0 = wave == 0;
            const auto rde = buffer_range(a.deta_part ? a.deta_part + rb * a.tplane + tokb + t0
                                                      : nullptr,
                                          w0 && a.deta_part ? 4u * len : 0u);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(de), rde,
                                                  4 * (g == 0 ? c : kSub), 0, 0);
            const auto rdv = buffer_range(static_cast<TIO*>(a.dV) + (tokb + t0) * D,
                                          w0 ? (uint32_t)(len * D * sizeof(TIO)) : 0u);
            buffer_store4(rdv, (c * D + r0 + 4 * g) * (int)sizeof(TIO), -dE, TIO{});
        }
        // dA = -(F^T dZ) o U: A = RL(F^T) = CL(F) registers, B = CL(dZ_blk)
        f32x4 dA = mmt<BF, true, true>(F, dZb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int v = 0; v < 4; ++v) dA[v] = (4 * g + v <= c) ? -dA[v] : 0.f;
        put_cl<20>(L.dA[wave], 0, lane, dA);
        put_cl<20>(L.dE[wave], 0, lane, dE);
        if constexpr (MULTI) put_cl<20>(L.F[wave], 0, lane, F);
        lds_order();
        if constexpr (MULTI) {
            // H = W - G_{<sigma}: add this sub-tile's update back
            const f32x4 Fa = rl<20>(L.F[wave], 0, lane);
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb)
                Hr[bb] = mmt<BF, false, true>(Fa, cl<S>(L.K, 16 * blk(bb), lane), Hr[bb]);
        }
        const f32x4 dAa = rl<20>(L.dA[wave], 0, lane);   // RL(dA)
        const f32x4 dEa = rl<20>(L.dE[wave], 0, lane);   // RL(dE)
        f32x4 Fn;
#pragma unroll
        for (int v = 0; v < 4; ++v) Fn[v] = -F[v];
        const uint32_t tile_bytes = (uint32_t)(len * D * sizeof(float));
        const auto rdk = buffer_range(a.dK_part + rb * a.plane + (tokb + t0) * D, tile_bytes);
        const auto rdq = buffer_range(a.dQ_part + rb * a.plane + (tokb + t0) * D, tile_bytes);
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            const int b = blk(bb);
            const f32x4 kc = cl<S>(L.K, 16 * b, lane);
            const f32x4 qc = cl<S>(L.Q, 16 * b, lane);
            const f32x4 wc = cl<S>(L.W, 16 * b, lane);
            // dK (tokens x dims) = -F^T P + dE^T W + dA Q   (P: this sub-tile's, CL)
            f32x4 dK = mm2<BF>(Fn, P[bb], dE, wc, f32x4{0.f, 0.f, 0.f, 0.f});
            dK = mmt<BF, true, true>(dAa, qc, dK);
            // dQ (tokens x dims) = dZ^T H + dA^T K
            f32x4 dQ;
            if constexpr (MULTI) dQ = mm2<BF>(dZb, Hr[bb], dA, kc, f32x4{0.f, 0.f, 0.f, 0.f});
            else dQ = mm2<BF>(dZb, wc, dA, kc, f32x4{0.f, 0.f, 0.f, 0.f});
            // token 4g + v of the sub-tile, column 16b + c; rows past len dropped
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int off = 4 * ((4 * g + v) * D + 16 * b + c);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(dK[v]), rdk, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(dQ[v]), rdq, off, 0, 0);
            }
            // P += dZ Q, dW += dE K
            P[bb] = mmt<BF, true, true>(dZa, qc, P[bb]);
            dWa[bb] = mmt<BF, false, true>(dEa, kc, dWa[bb]);
        }
        if (si == 0) {   // the chunk is done: its dW is the previous chunk's dW_next
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb) {
                P[bb] += dWa[bb];
                dWa[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    // The sub-tiles after the segment only carry the state's cotangent back to the
    // segment's end, dW_c = dW_{c+1} (I - K diag(eta) K^T) + dZ U^T: the P chain of
    // the full step below, the same operations in the same order (so the result has
    // the bits the unsegmented pass reaches there), without E, the gradients of
    // K, Q, V, eta or the state.  One sub-tile per chunk (nseg > 1 only then).
    auto cot_step = [&](int j, auto slot) {
        auto& cur = bufs[decltype(slot)::value];
        auto& nxt = bufs[decltype(slot)::value ^ 1];
        __syncthreads();   // the previous sub-tile's tiles are consumed
        put(cur, true, false);
        const float et = cur.eta_ok ? cur.eta : 0.f;
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) put_cl<S>(L.P, 16 * blk(bb), lane, P[bb]);
        __syncthreads();
        fetch(nxt, j - 1, true, j - 1 <= j_hi);   // j > j_hi >= j_lo
        f32x4 PKw = {0.f, 0.f, 0.f, 0.f}, Sw = PKw;
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            const int b = blk(bb);
            const f32x4 kb = rl<S>(L.K, 16 * b, lane);
            PKw = mmt<BF, false, true>(rl<S>(L.P, 16 * b, lane), kb, PKw);
            Sw = mmt<BF, true, true>(kb, rl<S>(L.Q, 16 * b, lane), Sw);
        }
        put_cl<20>(L.part[wave][1], 0, lane, PKw);
        put_cl<20>(L.part[wave][2], 0, lane, Sw);
        __syncthreads();
        const f32x4 PK = reduce(1), Sm = reduce(2);
        f32x4 Mk;
#pragma unroll
        for (int v = 0; v < 4; ++v) Mk[v] = (4 * g + v <= c) ? Sm[v] : 0.f;
        put_cl<20>(L.M[wave], 0, lane, Mk);
        lds_order();
        const f32x4 dZa = cl<20>(L.dZ, 0, lane);
        f32x4 dF = mmt<BF, true, false>(dZa, rl<20>(L.M[wave], 0, lane), f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 dE;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            dF[v] = -dF[v] - PK[v];
            dE[v] = dF[v] * et;
        }
        put_cl<20>(L.dE[wave], 0, lane, dE);
        lds_order();
        const f32x4 dEa = rl<20>(L.dE[wave], 0, lane);
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            const int b = blk(bb);
            P[bb] = mmt<BF, true, true>(dZa, cl<S>(L.Q, 16 * b, lane), P[bb]);
            dWa[bb] = mmt<BF, false, true>(dEa, cl<S>(L.K, 16 * b, lane), dWa[bb]);
        }
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb) {
            P[bb] += dWa[bb];
            dWa[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    fetch(bufs[0], last, true, last <= j_hi && opens(last));
    if constexpr (!SEG) {   // one segment
        int j = last;
        for (; j >= 1; j -= 2) {
            rev_step(j, slot0);
            rev_step(j - 1, slot1);
        }
        if (j == 0) rev_step(0, slot0);
    } else {
        int j = last;
        for (; j >= j_lo + 1; j -= 2) {
            if (j > j_hi) cot_step(j, slot0);
            else rev_step(j, slot0);
            if (j - 1 > j_hi) cot_step(j - 1, slot1);
            else rev_step(j - 1, slot1);
        }
        if (j == j_lo) rev_step(j_lo, slot0);
    }
    if (j_lo == 0) {
        float* dW0 = a.dW0 + ((size_t)slice * D + r0) * D;
#pragma unroll
        for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
            for (int v = 0; v < 4; ++v) dW0[(4 * g + v) * D + 16 * blk(bb) + c] = P[bb][v];
    }
}

// n floats set to zero: 16-byte stores (n a multiple of 4, p 16-byte aligned)
// or, with VEC false, 4-byte ones
// dK and dQ: the row-block planes added in order, four elements per thread,
// written in the I/O type
template <typename TIO, int NB>
__global__ __launch_bounds__(256) void sum_planes_kernel(const float* __restrict__ dK_part,
                                                         const float* __restrict__ dQ_part,
                                                         TIO* __restrict__ dK, TIO* __restrict__ dQ,
                                                         size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    auto put = [](TIO* out, size_t i, f32x4 v) {
        if constexpr (sizeof(TIO) == 4) {
            reinterpret_cast<f32x4*>(out)[i] = v;
        } else {
            const u32x2 p = pack_bf16x4(v);
            reinterpret_cast<uint2*>(out)[i] = uint2{p.x, p.y};
        }
    };
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n / 4; i += stride) {
        f32x4 k = reinterpret_cast<const f32x4*>(dK_part)[i];
        f32x4 q = reinterpret_cast<const f32x4*>(dQ_part)[i];
#pragma unroll
        for (int r = 1; r < NB; ++r) {
            k += reinterpret_cast<const f32x4*>(dK_part + r * n)[i];
            q += reinterpret_cast<const f32x4*>(dQ_part + r * n)[i];
        }
        put(dK, i, k);
        put(dQ, i, q);
    }
}

// deta: the row-block planes added in order (deta is only 4-byte aligned)
template <int NB>
__global__ __launch_bounds__(256) void sum_deta_kernel(const float* __restrict__ part,
                                                       float* __restrict__ deta, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float v = part[i];
#pragma unroll
        for (int r = 1; r < NB; ++r) v += part[r * n + i];
        deta[i] = v;
    }
}

unsigned elementwise_grid(size_t n)
{
    return (unsigned)std::min<size_t>((n / 4 + 255) / 256, 4096);
}

// Segments along T for chunks of at most one sub-tile when the (sequence, row
// block) units leave compute units idle.  Segment k (sub-tiles b_k .. b_{k+1}-1 of
// N) recomputes the forward over b_{k+1} sub-tiles, carries the cotangent back over
// N - b_{k+1} and runs the full reverse over its own b_{k+1} - b_k, at relative
// costs kFwd, kCot and kRev per sub-tile.  Equal costs give b_{k+1} = N s_k /
// s_{S-1}, s_k = sum_{i <= k} r^i, r = kRev / (kFwd - kCot + kRev).  The ratios are
// fitted to where the two-segment split of 1 x 32 heads, T = 32768 (bf16, d = 64)
// is fastest: b_1 / N = 0.23, 0.41, 0.47, 0.535, 0.59 measured 5.00, 4.33, 4.12,
// 4.32 and 4.50 ms per call (one segment: 5.00 ms; every split gives the same bits);
// with four segments the same ratios stay best (3.82 ms; kCot = 0, 0.5, 0.7: 4.18,
// 4.23, 4.88).  Segments per sequence at 128 units: 2 -> 4.12, 4 -> 3.85,
// 6 -> 3.91, 8 -> 4.22 ms; one wave per unit instead of two: 4.96 (2), 4.26 (4).
constexpr double kFwd = 0.15, kCot = 0.25, kRev = 1.0;
constexpr int kMinBwdSegSub = 64;   // shortest segment, in sub-tiles

void bwd_segments(long wave_units, int nsubtiles, int& nseg, int* bound)
{
    for (int i = 0; i <= kMaxBwdSeg; ++i) bound[i] = 0;
    // at most four waves of segment units per compute unit (wave_units: units times
    // waves per unit): 1 x 32 heads (128 two-wave units) takes four segments, 8 x 12
    // heads (384 one-wave units) two (0.515 -> 0.497 ms)
    long S = std::min<long>(kMaxBwdSeg, 4 * kComputeUnits / std::max<long>(wave_units, 1));
    S = std::min<long>(S, nsubtiles / kMinBwdSegSub);
    nseg = S > 1 ? (int)S : 1;
    if (nseg == 1) return;
    const double r = kRev / (kFwd - kCot + kRev);
    double sk[kMaxBwdSeg];
    double acc = 0.0, term = 1.0;
    for (int k = 0; k < nseg; ++k) {
        acc += term;
        sk[k] = acc;
        term *= r;
    }
    bound[0] = 0;
    for (int k = 0; k + 1 < nseg; ++k) {
        const int e = (int)(nsubtiles * sk[k] / sk[nseg - 1] + 0.5);
        bound[k + 1] = std::max(bound[k] + 1, std::min(e, nsubtiles - (nseg - 1 - k)));
    }
    bound[nseg] = nsubtiles;
}

template <typename TIO, int D>
hipError_t launch_typed(const LinearBwdArgs& a, hipStream_t s)
{
    constexpr int NB = D / 16;
    const int nch = (a.T + a.chunk - 1) / a.chunk;
    const size_t n = (size_t)a.BH * a.T * D, ntok = (size_t)a.BH * a.T;
    char* ws = static_cast<char*>(a.workspace);
    BwdArgs k;
    k.K = a.K; k.Q = a.Q; k.V = a.V; k.eta = a.eta; k.eta_scalar = a.eta_scalar;
    k.W0 = a.W0; k.dZ = a.dZ; k.dWT = a.dW_T; k.dV = a.dV; k.dW0 = a.dW0;
    k.states = reinterpret_cast<float*>(ws);
    ws += linear_bwd_align((size_t)a.BH * (nch + 1) * D * D * sizeof(float));
    // dK, dQ and deta are sums over the d/16 row blocks: one fp32 plane each per row
    // block, added in order after the scan
    k.plane = n;
    k.tplane = ntok;
    k.dK_part = reinterpret_cast<float*>(ws);
    ws += linear_bwd_align(NB * n * sizeof(float));
    k.dQ_part = reinterpret_cast<float*>(ws);
    ws += linear_bwd_align(NB * n * sizeof(float));
    k.deta_part = a.deta ? reinterpret_cast<float*>(ws) : nullptr;
    k.BH = a.BH; k.T = a.T; k.chunk = a.chunk;
    constexpr bool F32 = sizeof(TIO) == 4;
    // waves per unit: at d = 64 with bf16 I/O two while the units leave compute
    // units idle, else one; otherwise fixed per d
    const int nw = (!F32 && D == 64) ? ((long)a.BH * NB >= kComputeUnits ? 1 : 2) : bwd_waves<D>();
    bwd_segments((long)a.BH * NB * nw, a.chunk <= kSub ? nch : 0, k.nseg, k.bound);
    const unsigned grid = (unsigned)(((a.BH + 7) / 8) * 8 * NB * k.nseg);
    auto launch = [&](auto nw) {
        constexpr int NW = decltype(nw)::value;
        if (a.chunk > kSub)
            hipLaunchKernelGGL((linear_bwd_kernel<TIO, D, NW, true>), dim3(grid), dim3(64 * NW), 0,
                               s, k);
        else if (k.nseg > 1)
            hipLaunchKernelGGL((linear_bwd_kernel<TIO, D, NW, false, true>), dim3(grid),
                               dim3(64 * NW), 0, s, k);
        else
            hipLaunchKernelGGL((linear_bwd_kernel<TIO, D, NW, false>), dim3(grid), dim3(64 * NW),
                               0, s, k);
    };
    if constexpr (!F32 && D == 64) {
        if (nw == 1) launch(std::integral_constant<int, 1>{});
        else launch(std::integral_constant<int, 2>{});   // two waves per unit
    } else {
        launch(std::integral_constant<int, bwd_waves<D>()>{});
    }
    hipLaunchKernelGGL((sum_planes_kernel<TIO, NB>), dim3(elementwise_grid(n)), dim3(256), 0, s,
                       (const float*)k.dK_part, (const float*)k.dQ_part, static_cast<TIO*>(a.dK),
                       static_cast<TIO*>(a.dQ), n);
    if (a.deta)
        hipLaunchKernelGGL((sum_deta_kernel<NB>), dim3(elementwise_grid(4 * ntok)), dim3(256), 0,
                           s, (const float*)k.deta_part, a.deta, ntok);
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_dtype(const LinearBwdArgs& a, hipStream_t s)
{
    switch (a.d) {
    case 16: return launch_typed<TIO, 16>(a, s);
    case 32: return launch_typed<TIO, 32>(a, s);
    case 64: return launch_typed<TIO, 64>(a, s);
    case 128: return launch_typed<TIO, 128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t linear_bwd_align(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

size_t linear_bwd_workspace(int BH, int T, int d, int chunk, bool bf16)
{
    (void)bf16;
    const size_t nch = (size_t)(T + chunk - 1) / chunk;
    const size_t n = (size_t)BH * T * d, nb = (size_t)d / 16;
    // chunk-start states, then the row blocks' fp32 planes of dK, dQ and deta
    return linear_bwd_align((size_t)BH * (nch + 1) * d * d * sizeof(float)) +
           2 * linear_bwd_align(nb * n * sizeof(float)) +
           linear_bwd_align(nb * (size_t)BH * T * sizeof(float));
}

hipError_t launch_linear_bwd(const LinearBwdArgs& a, hipStream_t s)
{
    return a.bf16 ? launch_dtype<uint16_t>(a, s) : launch_dtype<float>(a, s);
}

}  // namespace ttt
