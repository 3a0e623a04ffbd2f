// TTT-Linear forward scan on gfx950 matrix cores (bf16 operands, fp32 state).
//
// Method: PaperTrace "5 · TestingTime 训练与长上下文" §1.1/§2.3 (chunked update,
// gradient of 1/2||W k - v||^2 at the chunk-start state, inclusive read), in the
// dual form of diosapp "Test-Time Training (TTT) guide" §3.  For a 16-token
// sub-tile with tokens as columns:
//     E = W_c K - V                 (gradient factor, at the chunk-start state)
//     Z = M Q - E diag(eta) triu(K^T Q)
//     M = M - E diag(eta) K^T       (running state; W_{c+1} = M at chunk end)
// For chunk <= 16 a sub-tile is one chunk (W_c = M); for a chunk that is a
// multiple of 16, E keeps using the frozen chunk-start W_c while M runs.
//
// Work split.  Row i of Z and of the state depends only on row i of W0 and
// feature i of V (and on all of K, Q, eta), so each wave owns 16 output rows of
// one (batch, head) and never talks to another wave.  The d/16 waves of a head
// are placed on one XCD so that they share that XCD's L2 for K and Q.
//
// Register dataflow (one wave; see mfma_common.h for the MFMA layouts).
//   M      : d/16 fp32 C/D tiles; tile jb, lane (o, g), value i holds
//            W[o][pi(jb, 4g+i)] with pi(2m, 4g+i) = 32m+8g+i and
//            pi(2m+1, 4g+i) = 32m+8g+4+i, so that the bf16 x32-operand of step
//            m is (tile 2m, tile 2m+1) packed, and K/Q rows load as 16 bytes.
//   E^T    = K^T W^T - V^T      : A = K rows (lane = token), B = W rows; C from
//            -V^T, which an identity product moves into C/D layout.
//   F      = -diag(eta) E^T in bf16 (C/D layout = B operand over tokens).
//   M_jb  += Kt_jb F            : Kt_jb = K tile transposed by an identity
//            product (lane = input feature, slots = tokens).
//   S^T    = K^T Q masked s<=t  : C/D layout = B operand over tokens.
//   Z^T    = W Q^T + F^T... :  A = W rows, B = Q rows, then A = F read as
//            (E diag(-eta)) rows, B = S^T; lane (t, g) ends with Z[t][4g..4g+3].
// No LDS, no barriers, no atomics.
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int kStep = 16;

// eta modes: none (scalar for every token), per-token scalar loads, per-token
// 16-byte loads (every sub-tile full and the eta rows 16-byte aligned)
enum { kEtaScalar = 0, kEtaToken = 1, kEtaToken4 = 2 };

template <int D, int RB = 1>
struct Tile {
    u32x4 k[D / 32];   // K row (lane = token), 16-byte pieces at 32m + 8g
    u32x4 q[D / 32];   // Q row, same pieces
    u32x2 v[RB];       // V[token][out0 + 16r + 4g .. +3] for the wave's RB row blocks
    f32x4 eta;         // eta of tokens 4g .. 4g+3 (C/D rows), raw
    int n;             // valid tokens (0 = past the end)
};

// Loads a sub-tile exactly as stored.  Rows past the sub-tile's last valid token
// re-read a valid row of the same slice (addresses stay in bounds); they are
// neutralised later by giving them eta = 0, so no select ever touches the
// loaded registers here (a select on load results would force the wait for the
// load at the point of the select and stall the prefetch pipeline).
template <int D, int ETA, bool FULL, int RB = 1>
__device__ __forceinline__ void load_tile(Tile<D, RB>& t, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ Q,
                                          const uint16_t* __restrict__ V,
                                          const float* __restrict__ eta,
                                          size_t tok0, int s0, int n, int out0, int lane)
{
    const int c = lane & 15, g = lane >> 4;
    t.n = n;
    const size_t row = (tok0 + s0 + (FULL || c < n ? c : 0)) * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
        t.k[m] = *(const u32x4*)(K + row + 32 * m + 8 * g);
        t.q[m] = *(const u32x4*)(Q + row + 32 * m + 8 * g);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) t.v[r] = *(const u32x2*)(V + row + out0 + 16 * r + 4 * g);
    if (ETA == kEtaToken4) {
        t.eta = *(const f32x4*)(eta + tok0 + s0 + 4 * g);
    } else if (ETA == kEtaToken) {
        const float* e = eta + tok0 + s0;
        t.eta.x = e[FULL || 4 * g + 0 < n ? 4 * g + 0 : 0];
        t.eta.y = e[FULL || 4 * g + 1 < n ? 4 * g + 1 : 0];
        t.eta.z = e[FULL || 4 * g + 2 < n ? 4 * g + 2 : 0];
        t.eta.w = e[FULL || 4 * g + 3 < n ? 4 * g + 3 : 0];
    }
}

// One slice's K, Q, V, eta and Z as buffer resources, with this lane's byte
// offset within a 16-token tile: K and Q row c at features 8g (+ 32m), V and Z row
// c at the wave's features out0 + 4g (+ 16r), eta 4g.  Loads and stores of whole
// tiles then put the tile's start in the scalar offset and need no vector address
// arithmetic.  The buffer's range check is not relied on (on gfx9 it covers the
// vector offset only): only tiles inside the slice are addressed this way, and
// the slice must span less than 2^31 bytes (T d 2) so that offsets fit.
struct SliceBuffers {
    __amdgpu_buffer_rsrc_t k, q, v, e, z;
    int kq, vo, eo;
};

constexpr int kRawBufferFlags = 0x00020000;   // dword 3 of a gfx9 buffer resource: raw 32-bit data

template <int D>
__device__ __forceinline__ SliceBuffers slice_buffers(const uint16_t* K, const uint16_t* Q,
                                                      const uint16_t* V, const float* eta,
                                                      uint16_t* Z, size_t tok0, int T, int out0,
                                                      int lane)
{
    const int c = lane & 15, g = lane >> 4;
    const int bytes = (int)min((long long)T * D * 2, 0x7fffffffLL);
    SliceBuffers b;
    b.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(K + tok0 * D), 0, bytes,
                                            kRawBufferFlags);
    b.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Q + tok0 * D), 0, bytes,
                                            kRawBufferFlags);
    b.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(V + tok0 * D), 0, bytes,
                                            kRawBufferFlags);
    b.z = __builtin_amdgcn_make_buffer_rsrc(Z + tok0 * D, 0, bytes, kRawBufferFlags);
    b.e = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(eta ? eta + tok0 : nullptr), 0,
                                            eta ? T * 4 : 0, kRawBufferFlags);
    b.kq = (c * D + 8 * g) * 2;
    b.vo = (c * D + out0 + 4 * g) * 2;
    b.eo = 16 * g;
    return b;
}

// load_tile for a whole tile starting at token s0 of the slice (inside it)
template <int D, int ETA, int RB>
__device__ __forceinline__ void load_tile_full(Tile<D, RB>& t, const SliceBuffers& b, int s0)
{
    const int so = s0 * D * 2;
    t.n = 16;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
        t.k[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b.k, b.kq + 64 * m, so, 0));
        t.q[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b.q, b.kq + 64 * m, so, 0));
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
        t.v[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(b.v, b.vo + 32 * r, so, 0));
    if (ETA == kEtaToken4) {
        t.eta = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.e, b.eo, s0 * 4, 0));
    } else if (ETA == kEtaToken) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            t.eta[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(b.e, b.eo + 4 * i, s0 * 4, 0));
    }
}

// K of one sub-tile, re-laid out in LDS as d/16 row-major 16 x 16 bf16 blocks
// (block jb holds K[token][pi(jb, 0..15)], 512 bytes), then read back with the
// gfx950 transpose read: in each 16-lane group, lanes 4r..4r+3 supply row r
// (4 elements each) and lane i receives element i of rows 0..3.  Reading block
// jb at (8 * lane) therefore gives lane (i, g) the four tokens 4g..4g+3 of input
// feature pi(jb, i): the A operand of the state update, already in bf16.
template <int D, int RB>
__device__ __forceinline__ void transpose_k(u32x2 (&kt)[D / 16], const Tile<D, RB>& t, u32x2* lds,
                                            int lane)
{
    const int c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
        lds[(2 * m) * 64 + 4 * c + g] = lo_half(t.k[m]);
        lds[(2 * m + 1) * 64 + 4 * c + g] = hi_half(t.k[m]);
    }
    asm volatile("" ::: "memory");   // keep the reads after the writes (one wave: LDS is in order)
#pragma unroll
    for (int jb = 0; jb < D / 16; ++jb) {
        auto p = (__attribute__((address_space(3))) s16x4*)(lds + jb * 64 + lane);
        kt[jb] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
    }
    asm volatile("" ::: "memory");
}

// The same transpose into the upper halves of 32-deep operands whose lower halves
// stay zero: [0 | K^T] [I ; F] is the 16-deep product K^T F, and tuples that live
// across the loop keep their zeros without a move per product.
template <int D, int RB>
__device__ __forceinline__ void transpose_k_hi(u32x4 (&ktz)[D / 16], const Tile<D, RB>& t,
                                               u32x2* lds, int lane)
{
    u32x2 kt[D / 16];
    transpose_k<D>(kt, t, lds, lane);
#pragma unroll
    for (int jb = 0; jb < D / 16; ++jb) {
        ktz[jb].z = kt[jb].x;
        ktz[jb].w = kt[jb].y;
    }
}

// The unit is one (batch, head) sequence and one 16-row block of its state.
template <int D, int PF, int WPB, int ETA, bool FULL, bool MULTI>
__global__ __launch_bounds__(64 * WPB) void linear_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, int BH, int T, int chunk)
{
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    __shared__ u32x2 lds_all[WPB * NB * 64];

    // WPB waves per workgroup own WPB consecutive 16-row slices of one unit
    // (a workgroup's waves sit on distinct SIMDs of one CU and share its L1)
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    u32x2* lds_kt = lds_all + wave * NB * 64;
    int slice, bpart;
    xcd_unit_part(blockIdx.x, NB / WPB, slice, bpart);
    const int ob = bpart * WPB + wave;
    if (slice >= BH) return;
    const int out0 = ob * 16;
    const size_t tok0 = (size_t)slice * T;

    // state rows out0 + c, columns pi(jb, 4g + i)
    f32x4 M[NB];
    {
        const float* w = W0 + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[2 * m] = *(const f32x4*)(w + 32 * m + 8 * g);
            M[2 * m + 1] = *(const f32x4*)(w + 32 * m + 8 * g + 4);
        }
    }
    const u32x2 I16 = identity_b16(lane);

    const int step = chunk < kStep ? chunk : kStep;
    const int ntiles = (T + step - 1) / step;
    const int tiles_per_chunk = chunk / step;   // 1 when chunk <= 16

    Tile<D> buf[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int s0 = p * step;
        const int n = s0 < T ? min(step, T - s0) : 0;
        load_tile<D, ETA, FULL>(buf[p], K, Q, V, eta, tok0, n > 0 ? s0 : 0, n, out0, lane);
    }
    u32x2 kt[NB];   // transposed K of the current sub-tile
    transpose_k<D>(kt, buf[0], lds_kt, lane);

    u32x4 Wc[NM];   // bf16 chunk-start state (operand of E)
    int in_chunk = 0;
    for (int tau0 = 0; tau0 < ntiles; tau0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int tau = tau0 + p;
            if (tau >= ntiles) break;
            Tile<D> cur = buf[p];
            {
                const int s0 = (tau + PF) * step;
                const int n = s0 < T ? min(step, T - s0) : 0;
                load_tile<D, ETA, FULL>(buf[p], K, Q, V, eta, tok0, n > 0 ? s0 : 0, n, out0,
                                        lane);
            }
            const int s0 = tau * step;
            // eta of padding tokens (4g + i >= n) is zero: they then add nothing
            // to E diag(eta) K^T or to the E diag(eta) S term of Z
            f32x4 et = ETA == kEtaScalar ? f32x4{eta_scalar, eta_scalar, eta_scalar, eta_scalar}
                                         : cur.eta;
            if (!FULL) {
                et.x = (4 * g + 0 < cur.n) ? et.x : 0.f;
                et.y = (4 * g + 1 < cur.n) ? et.y : 0.f;
                et.z = (4 * g + 2 < cur.n) ? et.z : 0.f;
                et.w = (4 * g + 3 < cur.n) ? et.w : 0.f;
            }
            // running state in bf16 (operand of W Q, and of E at a chunk start)
            u32x4 Mf[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) Mf[m] = pack_bf16x8(M[2 * m], M[2 * m + 1]);
            if (!MULTI || in_chunk == 0) {
#pragma unroll
                for (int m = 0; m < NM; ++m) Wc[m] = Mf[m];
            }
            if (MULTI) in_chunk = (in_chunk + 1 == tiles_per_chunk) ? 0 : in_chunk + 1;
            // E^T = K^T W_c^T - V^T
            const u32x2 vneg = cur.v[0] ^ u32x2{0x80008000u, 0x80008000u};
            f32x4 Et = mfma16(vneg, I16, f32x4{0, 0, 0, 0});
#pragma unroll
            for (int m = 0; m < NM; ++m) Et = mfma32(cur.k[m], Wc[m], Et);
            // F = -diag(eta) E^T  (bf16)
            const u32x2 F = pack_bf16x4(-et * Et);
            // M += K F, block by block (contraction over the sub-tile's tokens)
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) M[jb] = mfma16(kt[jb], F, M[jb]);
            // S^T = K^T Q with the inclusive causal mask s <= t
            f32x4 St = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) St = mfma32(cur.k[m], cur.q[m], St);
            f32x4 Sm;
            Sm.x = (4 * g + 0 <= c) ? St.x : 0.f;
            Sm.y = (4 * g + 1 <= c) ? St.y : 0.f;
            Sm.z = (4 * g + 2 <= c) ? St.z : 0.f;
            Sm.w = (4 * g + 3 <= c) ? St.w : 0.f;
            const u32x2 Sb = pack_bf16x4(Sm);
            // Z^T = M Q^T - (E diag(eta)) S   (M as it was at the sub-tile start)
            f32x4 Zt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Zt = mfma32(Mf[m], cur.q[m], Zt);
            Zt = mfma16(F, Sb, Zt);
            if (FULL || c < cur.n) {
                const u32x2 zb = pack_bf16x4(Zt);
                *(u32x2*)(Z + (tok0 + s0 + c) * D + out0 + 4 * g) = zb;
            }
            // transposed K of the next sub-tile (its loads were issued PF-1 sub-tiles ago)
            if (tau + 1 < ntiles) transpose_k<D>(kt, buf[(p + 1) % PF], lds_kt, lane);
        }
    }

    float* w = W_out + (size_t)slice * D * D + (size_t)(out0 + c) * D;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        *(f32x4*)(w + 32 * m + 8 * g) = M[2 * m];
        *(f32x4*)(w + 32 * m + 8 * g + 4) = M[2 * m + 1];
    }
}

// Chunks of at most 16 tokens: every sub-tile is a chunk and the state feeds the
// next chunk's error directly.  The serial dependency W_c -> E_c -> W_{c+1} is cut
// short with
//     E_{c+1} = K_{c+1} W_{c+1}^T - V_{c+1}
//             = [K_{c+1} W_c^T - V_{c+1}] + (K_{c+1} K_c^T) F_c,   F_c = -diag(eta_c) E_c,
// (token-row layout; W_{c+1} = W_c + F_c^T K_c).  The bracket needs only the older
// state and the Gram matrix K_{c+1} K_c^T needs no state at all, so after F_c only
// one product stands between two chunks; the state update itself runs beside it.
//
// A wave owns RB consecutive 16-row blocks of the state (RB independent chains).
// They share the K/Q loads, the K transpose, the Gram matrix and the causal
// scores, and their chains interleave in one instruction stream, which measures
// faster than the same chains on separate waves of one compute unit.
template <int D, int PF, int WPB, int RB, int ETA, bool FULL>
__global__ __launch_bounds__(64 * WPB) void linear_mfma_chain_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ Q,
    const uint16_t* __restrict__ V, const float* __restrict__ eta, float eta_scalar,
    const float* W0, uint16_t* __restrict__ Z, float* W_out, int BH, int T_all, int chunk,
    const int* __restrict__ cu, int H, int total_T)
{
    constexpr int NB = D / 16;
    constexpr int NM = D / 32;
    static_assert(PF >= 2, "the next tile must be resident");
    static_assert(NB % (WPB * RB) == 0, "row blocks must tile the state");
    __shared__ u32x2 lds_all[WPB * NB * 64];

    // WPB waves per workgroup own WPB * RB consecutive 16-row blocks of one head
    // (a workgroup's waves sit on distinct SIMDs of one CU and share its L1)
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, g = lane >> 4;
    u32x2* lds_kt = lds_all + wave * NB * 64;
    int slice, bpart;
    xcd_unit_part(blockIdx.x, NB / (WPB * RB), slice, bpart);
    if (slice >= BH) return;
    const int out0 = (bpart * WPB + wave) * RB * 16;
    size_t tok0;
    int T;
    slice_span(cu, H, total_T, T_all, slice, tok0, T);
    if (T == 0) {   // an empty document: the state passes through
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const float* w = W0 + (size_t)slice * D * D + (size_t)(out0 + 16 * r + c) * D;
            float* wo = W_out + (size_t)slice * D * D + (size_t)(out0 + 16 * r + c) * D;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                *(f32x4*)(wo + 32 * m + 8 * g) = *(const f32x4*)(w + 32 * m + 8 * g);
                *(f32x4*)(wo + 32 * m + 8 * g + 4) = *(const f32x4*)(w + 32 * m + 8 * g + 4);
            }
        }
        return;
    }
    const int step = chunk;                    // <= 16
    const int ntiles = (T + step - 1) / step;

    f32x4 M[RB][NB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const float* w = W0 + (size_t)slice * D * D + (size_t)(out0 + 16 * r + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            M[r][2 * m] = *(const f32x4*)(w + 32 * m + 8 * g);
            M[r][2 * m + 1] = *(const f32x4*)(w + 32 * m + 8 * g + 4);
        }
    }
    const u32x2 I16 = identity_b16(lane);

    const SliceBuffers sres = slice_buffers<D>(K, Q, V, eta, Z, tok0, T, out0, lane);
    Tile<D, RB> buf[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int s0 = p * step;
        const int n = s0 < T ? min(step, T - s0) : 0;
        if constexpr (FULL) load_tile_full<D, ETA, RB>(buf[p], sres, n > 0 ? s0 : 0);
        else load_tile<D, ETA, FULL, RB>(buf[p], K, Q, V, eta, tok0, n > 0 ? s0 : 0, n, out0, lane);
    }

    // prologue: E_0 = K_0 W_0^T - V_0 directly
    u32x4 Mf[RB][NM];
    f32x4 Et[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
        for (int m = 0; m < NM; ++m) Mf[r][m] = pack_bf16x8(M[r][2 * m], M[r][2 * m + 1]);
        const u32x2 vneg = buf[0].v[r] ^ u32x2{0x80008000u, 0x80008000u};
        Et[r] = mfma16(vneg, I16, f32x4{0, 0, 0, 0});
#pragma unroll
        for (int m = 0; m < NM; ++m) Et[r] = mfma32(buf[0].k[m], Mf[r][m], Et[r]);
    }
    u32x4 ktz[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) ktz[jb] = u32x4{0u, 0u, 0u, 0u};
    transpose_k_hi<D>(ktz, buf[0], lds_kt, lane);
    u32x4 smz = {0u, 0u, 0u, 0u};   // causal scores in the upper half

    // One chunk.  Work for the next chunk (Gram term, bracket, transposed K, bf16
    // state) is done unconditionally: after the last chunk the next tile is a
    // valid re-read of this slice and its results are simply unused, so the
    // steady-state body has no branches for the scheduler to stop at.
    // `whole` (a compile-time tag) marks a tile known to hold 16 tokens: no masks
    // and no predicated store, so the step stays one basic block for the scheduler
    auto chunk_step = [&](const Tile<D, RB>& cur, const Tile<D, RB>& nxt, int tau, auto whole) {
        constexpr bool TF = FULL || decltype(whole)::value;
        const int s0 = tau * step;
        f32x4 et = ETA == kEtaScalar ? f32x4{eta_scalar, eta_scalar, eta_scalar, eta_scalar}
                                     : cur.eta;
        if (!TF) {
            et.x = (4 * g + 0 < cur.n) ? et.x : 0.f;
            et.y = (4 * g + 1 < cur.n) ? et.y : 0.f;
            et.z = (4 * g + 2 < cur.n) ? et.z : 0.f;
            et.w = (4 * g + 3 < cur.n) ? et.w : 0.f;
        }
        // F_c = -diag(eta) E_c (bf16): the only value the next chunk waits for
        u32x4 IF[RB];   // [I ; F_c]
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const u32x2 F = pack_bf16x4(-et * Et[r]);
            IF[r] = u32x4{I16.x, I16.y, F.x, F.y};
        }
        // E_{c+1} = K_{c+1} W_c^T + [-V_{c+1} | G_c] [I ; F_c]
        {
            f32x4 Gt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Gt = mfma32(cur.k[m], nxt.k[m], Gt);
            const u32x2 G = pack_bf16x4(Gt);   // A operand of K_{c+1} K_c^T
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                f32x4 P = {0, 0, 0, 0};
#pragma unroll
                for (int m = 0; m < NM; ++m) P = mfma32(nxt.k[m], Mf[r][m], P);
                const u32x2 vneg = nxt.v[r] ^ u32x2{0x80008000u, 0x80008000u};
                Et[r] = mfma32(u32x4{vneg.x, vneg.y, G.x, G.y}, IF[r], P);
            }
        }
        // W_{c+1} = W_c + F_c^T K_c, block by block
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) M[r][jb] = mfma32(ktz[jb], IF[r], M[r][jb]);
        // Z_c = Q_c W_c^T - causal (eta-weighted) scores times E_c
        f32x4 St = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NM; ++m) St = mfma32(cur.k[m], cur.q[m], St);
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
        for (int r = 0; r < RB; ++r) {
            f32x4 Zt = {0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < NM; ++m) Zt = mfma32(Mf[r][m], cur.q[m], Zt);
            Zt = mfma32(IF[r], smz, Zt);   // + [I | F_c^T] [0 ; scores]
            if constexpr (FULL) {
                __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(Zt), sres.z, sres.vo + 32 * r,
                                                      s0 * D * 2, 0);
            } else if (TF || c < cur.n) {
                const u32x2 zb = pack_bf16x4(Zt);
                *(u32x2*)(Z + (tok0 + s0 + c) * D + out0 + 16 * r + 4 * g) = zb;
            }
        }
        transpose_k_hi<D>(ktz, nxt, lds_kt, lane);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int m = 0; m < NM; ++m) Mf[r][m] = pack_bf16x8(M[r][2 * m], M[r][2 * m + 1]);
    };
    auto refill = [&](Tile<D, RB>& slot, int tau) {
        const int s1 = tau * step;
        const int n = s1 < T ? min(step, T - s1) : 0;
        if constexpr (FULL) load_tile_full<D, ETA, RB>(slot, sres, n > 0 ? s1 : 0);
        else load_tile<D, ETA, FULL, RB>(slot, K, Q, V, eta, tok0, n > 0 ? s1 : 0, n, out0, lane);
    };
    // a tile known to hold 16 tokens: unclamped loads
    auto refill_whole = [&](Tile<D, RB>& slot, int tau) {
        load_tile<D, ETA, true, RB>(slot, K, Q, V, eta, tok0, tau * step, 16, out0, lane);
    };

    const std::integral_constant<bool, true> whole;
    const std::integral_constant<bool, false> ragged;
    int tau0 = 0;
    if constexpr (!FULL) {
        // ragged sequences of 16-token chunks: every tile before the last partial
        // one is whole (loads stay clamped, as they may reach the partial tile)
        const int nwhole = step == 16 ? T / 16 : 0;
        for (; tau0 + 2 * PF <= nwhole; tau0 += PF) {   // the refills are whole too
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                chunk_step(buf[p], buf[(p + 1) % PF], tau0 + p, whole);
                refill_whole(buf[p], tau0 + p + PF);
            }
        }
        for (; tau0 + PF <= nwhole; tau0 += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                chunk_step(buf[p], buf[(p + 1) % PF], tau0 + p, whole);
                refill(buf[p], tau0 + p + PF);
            }
        }
    }
    for (; tau0 + PF <= ntiles; tau0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            chunk_step(buf[p], buf[(p + 1) % PF], tau0 + p, ragged);
            refill(buf[p], tau0 + p + PF);
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        if (tau0 + p >= ntiles) break;
        chunk_step(buf[p], buf[(p + 1) % PF], tau0 + p, ragged);
    }

#pragma unroll
    for (int r = 0; r < RB; ++r) {
        float* w = W_out + (size_t)slice * D * D + (size_t)(out0 + 16 * r + c) * D;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            *(f32x4*)(w + 32 * m + 8 * g) = M[r][2 * m];
            *(f32x4*)(w + 32 * m + 8 * g + 4) = M[r][2 * m + 1];
        }
    }
}

// Launch choices, all measured on MI355X (256 compute units):
//  - prefetch depth of the chunk-16 kernel: 8 chunks (1x32 heads x 32768 tokens:
//    605 -> 438 us against 4), 4 where the registers do not allow 8;
//  - past 256 (head, 16-row block) units, the shared-tile kernel (d = 64, 128)
//    or two row blocks per wave take over from one wave per unit.
constexpr int kChainPrefetch = 8;
constexpr int kChainPrefetchWide = 4;
constexpr long kComputeUnits = 256;

// Chunks of several 16-token sub-tiles (E keeps the frozen chunk-start state).
template <int D, int WPB, int ETA, bool FULL>
void launch_multi(const LinearArgs& a, hipStream_t s)
{
    constexpr int PF = 4;
    const int units = (a.BH + 7) / 8 * 8;
    dim3 grid((unsigned)(units * (D / 16) / WPB)), block(64 * WPB);
    hipLaunchKernelGGL((linear_mfma_kernel<D, PF, WPB, ETA, FULL, true>), grid, block, 0, s,
                       (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta,
                       a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.BH, a.T, a.chunk);
}

template <int D, int RB, int ETA, bool FULL>
void launch_chain(const LinearArgs& a, hipStream_t s)
{
    // prefetch depth: 8 chunks where the registers allow it (d = 128 keeps 4)
    constexpr int PF = D * RB <= 64 ? kChainPrefetch : kChainPrefetchWide;
    const int units = (a.BH + 7) / 8 * 8;
    dim3 grid((unsigned)(units * (D / 16) / RB)), block(64);
    hipLaunchKernelGGL((linear_mfma_chain_kernel<D, PF, 1, RB, ETA, FULL>), grid, block, 0, s,
                       (const uint16_t*)a.K, (const uint16_t*)a.Q, (const uint16_t*)a.V, a.eta,
                       a.eta_scalar, a.W0, (uint16_t*)a.Z, a.W_out, a.BH, a.T, a.chunk, a.cu,
                       a.H, a.total_T);
}

template <int D, int ETA, bool FULL>
void launch_wpb(const LinearArgs& a, hipStream_t s)
{
    const long units = (long)a.BH * (D / 16);   // (batch*head, 16-row block) pairs
    if (a.chunk <= kStep) {
        // One wave per workgroup.  Measured on MI355X, a second wave on the same
        // compute unit slows both by 1.5-2x, so once the 16-row units outnumber
        // the 256 compute units a wave takes two of them (d <= 64).
        if constexpr (D <= 64) {
            if (units > kComputeUnits) {
                launch_chain<D, 2, ETA, FULL>(a, s);
                return;
            }
        }
        launch_chain<D, 1, ETA, FULL>(a, s);
        return;
    }
    // Two slices per workgroup when that still leaves at least 128 workgroups.
    if (units / 2 >= 128) launch_multi<D, 2, ETA, FULL>(a, s);
    else launch_multi<D, 1, ETA, FULL>(a, s);
}

template <int D>
hipError_t launch_d(const LinearArgs& a, hipStream_t s)
{
    if (a.cu) {   // packed documents: lengths known on the device only, chunk <= 16
        if (!a.eta) launch_wpb<D, kEtaScalar, false>(a, s);
        else launch_wpb<D, kEtaToken, false>(a, s);
        return hipGetLastError();
    }
    // every sub-tile holds 16 tokens: no padding logic at all
    // (whole-tile loads address a slice through 32-bit byte offsets)
    const bool full = a.chunk % kStep == 0 && a.T % kStep == 0 &&
                      (long long)a.T * a.d * 2 <= 0x7fffffffLL;
    const bool eta4 = a.eta && full && (reinterpret_cast<uintptr_t>(a.eta) % 16 == 0) &&
                      a.T % 4 == 0;
    if (full) {
        if (!a.eta) launch_wpb<D, kEtaScalar, true>(a, s);
        else if (eta4) launch_wpb<D, kEtaToken4, true>(a, s);
        else launch_wpb<D, kEtaToken, true>(a, s);
    } else {
        if (!a.eta) launch_wpb<D, kEtaScalar, false>(a, s);
        else launch_wpb<D, kEtaToken, false>(a, s);
    }
    return hipGetLastError();
}

}  // namespace

bool linear_mfma_supported(int d, int chunk, int bf16)
{
    return bf16 && (d == 32 || d == 64 || d == 128) && (chunk <= kStep || chunk % kStep == 0);
}

hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s)
{
    // Once the 16-row units outnumber the compute units, chunk-16 heads at d = 64
    // and 128 go to one workgroup per head that fetches K and Q once for all of
    // its waves (8x12 heads at d = 64: 49 us vs 52 us; at 32 heads, where every
    // unit has a compute unit to itself, the single-wave kernel is faster).  Packed
    // documents count one slice per (document, head).  That kernel's ragged form
    // (packed documents, or T not a multiple of 16) addresses a slice through 32-bit
    // buffer offsets, so it takes slices of fewer than 2^31 - 2^20 bytes.
    const long long span = a.cu ? a.total_T : a.T;
    const bool offsets_fit =
        (!a.cu && a.T % 16 == 0) || span * a.d * 2 < (1LL << 31) - (1LL << 20);
    if ((long)a.BH * (a.d / 16) > kComputeUnits && offsets_fit &&
        linear_coop_supported(a.d, a.chunk, a.bf16))
        return launch_linear_coop(a, s);
    switch (a.d) {
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ttt
