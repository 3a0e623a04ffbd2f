// gfx950 matrix-core helpers shared by the MFMA kernels.
//
// Register layouts of the 16x16 MFMA forms used here (wave64, lane l, lane
// group g = l / 16, c = l % 16):
//   A operand (16 x K): lane l holds row c, K-slots of group g;
//   B operand (K x 16): lane l holds column c, K-slots of group g;
//   C/D       (16x16) : lane l holds rows 4g + i (i = 0..3) of column c.
// Only the pairing of A-slot (g, j) with B-slot (g, j) matters for a product,
// so each kernel is free to choose which contraction index sits in which slot,
// as long as both operands use the same choice.  In particular a C/D tile,
// rounded to bf16, is directly a B operand (or, read as its transpose, an A
// operand) of a 16x16x16 product whose contraction index is the tile's row.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// D = A(16x16) B(16x16) + C, bf16 operands (4 per lane), fp32 accumulate.
// Issued as the 16x16x32 form with the upper four slots of both operands zero.
// The 16-deep forms (bf16 and fp16) read a stale accumulator when C is the result
// of a 16x16x32 MFMA issued just before them: a one-wave probe on gfx950 gives
// garbage for that pair back to back and the exact sum with 24 wait cycles
// between, and this toolchain emits no wait states for it (an accumulator
// written by the same 16-deep form, or the 16-deep product overwriting the
// 32-deep one's accumulator register, are fine).  Mixing the two depths in one
// dependent chain is what returned wrong results in the d = 128 kernels and, with
// the fp16 form, in the TTT-MLP kernel.  One depth everywhere avoids the pair; the
// zero slots add nothing.
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c)
{
    const u32x4 a8 = {a.x, a.y, 0u, 0u}, b8 = {b.x, b.y, 0u, 0u};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a8),
                                                  __builtin_bit_cast(bf16x8, b8), c, 0, 0, 0);
}

// D = A(16x32) B(32x16) + C, bf16 operands (8 per lane), fp32 accumulate.
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp16 forms of the same products (same rate as bf16; 11-bit significands)
__device__ __forceinline__ f32x4 mfma32h(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// (zero-padded 32-deep form, for the reason given at mfma16)
__device__ __forceinline__ f32x4 mfma16h(u32x2 a, u32x2 b, f32x4 c)
{
    const u32x4 a8 = {a.x, a.y, 0u, 0u}, b8 = {b.x, b.y, 0u, 0u};
    return mfma32h(a8, b8, c);
}

__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ u32x2 pack_f16x4(f32x4 v)
{
    return u32x2{pack_f16x2(v.x, v.y), pack_f16x2(v.z, v.w)};
}

__device__ __forceinline__ u32x4 pack_f16x8(f32x4 lo, f32x4 hi)
{
    return u32x4{pack_f16x2(lo.x, lo.y), pack_f16x2(lo.z, lo.w), pack_f16x2(hi.x, hi.y),
                 pack_f16x2(hi.z, hi.w)};
}

__device__ __forceinline__ f32x4 f16x4_to_f32(u32x2 v)
{
    return __builtin_convertvector(__builtin_bit_cast(f16x4, v), f32x4);
}

// 8 bf16 -> 8 fp16 (exact for magnitudes inside the fp16 normal range)
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pack_f16x2(__uint_as_float(v[i] << 16), __uint_as_float(v[i] & 0xffff0000u));
    return r;
}

// two fp32 -> packed bf16x2 (hardware convert, round to nearest even)
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 v)
{
    u32x2 r;
    r.x = pack_bf16x2(v.x, v.y);
    r.y = pack_bf16x2(v.z, v.w);
    return r;
}

// 8 bf16: slots 0..3 from `lo`, 4..7 from `hi`
__device__ __forceinline__ u32x4 pack_bf16x8(f32x4 lo, f32x4 hi)
{
    u32x4 r;
    r.x = pack_bf16x2(lo.x, lo.y);
    r.y = pack_bf16x2(lo.z, lo.w);
    r.z = pack_bf16x2(hi.x, hi.y);
    r.w = pack_bf16x2(hi.z, hi.w);
    return r;
}

__device__ __forceinline__ u32x2 lo_half(u32x4 v) { return u32x2{v.x, v.y}; }
__device__ __forceinline__ u32x2 hi_half(u32x4 v) { return u32x2{v.z, v.w}; }

// B operand of the 16x16 identity for a 16x16x16 product (slot (g, j) is
// contraction index 4g + j): multiplying a bf16 A operand by it moves the
// operand's 16x16 tile into C/D layout exactly (products by 1 and 0).
__device__ __forceinline__ u32x2 identity_b16(int lane)
{
    const int c = lane & 15, g = lane >> 4;
    const unsigned one = 0x3F80u;   // bf16 1.0
    unsigned e0 = (4 * g + 0 == c) ? one : 0u;
    unsigned e1 = (4 * g + 1 == c) ? one : 0u;
    unsigned e2 = (4 * g + 2 == c) ? one : 0u;
    unsigned e3 = (4 * g + 3 == c) ? one : 0u;
    return u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
}

// LDS 16x16 bf16 transpose through the gfx950 transpose read.  `x` is a tile
// in C/D layout converted to bf16 (lane (c, g) holds X[4g..4g+3][c]); it is
// stored as row c of a 512-byte block, and the transpose read (in each 16-lane
// group, lanes 4r..4r+3 supply row r and lane i receives element i of rows
// 0..3) returns lane (i, g) holding X[i][4g..4g+3]: the row index moves into the
// lane and the column index into the slots.  One wave; the caller keeps other
// waves off `block`.
__device__ __forceinline__ u32x2 lds_transpose16(u32x2* block, u32x2 x, int lane)
{
    block[4 * (lane & 15) + (lane >> 4)] = x;
    asm volatile("" ::: "memory");   // LDS is in order for one wave: read after the write
    auto p = (__attribute__((address_space(3))) s16x4*)(block + lane);
    u32x2 r = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
    asm volatile("" ::: "memory");
    return r;
}

// 16-token K and Q tiles staged in LDS (bf16, rows of d/8 16-byte granules).
// Granule gr of row r is stored at position gr ^ tile16_swizzle<D>(r).  Within
// each 16-lane group this spreads both reads of the tile over distinct banks
// (checked exhaustively for d = 64 and 128): the row read, lane (c, g) taking
// granule 4m + g of row c, and the transpose read, lane 4r + q of group g
// supplying 8 bytes of granule 4m + q of row 4g + r.  Lanes of different groups
// served in the same cycle can still meet: every lane of a transpose read takes
// the same 8-byte half of its granule, so 32 lanes reach only half the banks (a
// 2-way conflict that no granule permutation removes).
template <int D>
__device__ __forceinline__ int tile16_swizzle(int row)
{
    static_assert(D == 64 || D == 128, "swizzle defined for d = 64 and 128");
    if constexpr (D == 128) return ((row & 3) << 2) | (row >> 2);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 1) | (((row >> 3) & 1) << 1);
}

template <int D>
struct KQTile16 {
    u32x4 g[2][16 * (D / 8)];   // [K, Q][row * (D / 8) + swizzled granule]
};

// Workgroup index -> (unit, part) so that the `parts` workgroups of one unit run
// on the same XCD (workgroups are handed to the 8 XCDs round-robin), sharing
// that XCD's L2 for the unit's common inputs.  Grid = round_up(units, 8) * parts.
__device__ __forceinline__ void xcd_unit_part(int bid, int parts, int& unit, int& part)
{
    const int xcd = bid & 7, rest = bid >> 3;
    part = rest % parts;
    unit = (rest / parts) * 8 + xcd;
}

}  // namespace ttt
