// fp32 matrix-core tile helpers (v_mfma_f32_16x16x4_f32) over row-major fp32
// tiles.  Register forms of a 16 x 16 tile X (wave64, lane l, c = l % 16,
// g = l / 16, slot v = 0..3):
//   CL(X): lane holds X[4g + v][c]   (the MFMA result layout; a B operand whose
//                                     contraction index is X's row)
//   RL(X): lane holds X[c][4g + v]   (an A operand whose contraction index is
//                                     X's column)
// and RL(X) = CL(X^T).  mm16(RL(A), CL(B), CL(C)) = CL(A B + C) for 16 x 16 A, B.
#pragma once
#include <hip/hip_runtime.h>

#include "mfma_common.h"

namespace ttt {

// row-major fp32 with STRIDE floats per row (padding keeps the RL and CL reads
// of 16 lanes on distinct banks)
template <int STRIDE>
__device__ __forceinline__ f32x4 rl(const float* X, int col0, int lane)
{
    const int c = lane & 15, g = lane >> 4;
    return *reinterpret_cast<const f32x4*>(X + c * STRIDE + col0 + 4 * g);
}

template <int STRIDE>
__device__ __forceinline__ f32x4 cl(const float* X, int col0, int lane)
{
    const int c = lane & 15, g = lane >> 4;
    const float* p = X + (4 * g) * STRIDE + col0 + c;
    return f32x4{p[0], p[STRIDE], p[2 * STRIDE], p[3 * STRIDE]};
}

// write a CL register tile into columns col0..col0+15 of a row-major tile
template <int STRIDE>
__device__ __forceinline__ void put_cl(float* X, int col0, int lane, f32x4 v)
{
    const int c = lane & 15, g = lane >> 4;
    float* p = X + (4 * g) * STRIDE + col0 + c;
    p[0] = v[0];
    p[STRIDE] = v[1];
    p[2 * STRIDE] = v[2];
    p[3 * STRIDE] = v[3];
}

// keep the compiler from moving LDS accesses across this point (one wave: the
// LDS unit executes its accesses in order)
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// D += A B over a 16-wide contraction: A in RL form, B in CL form
__device__ __forceinline__ f32x4 mm16(f32x4 a, f32x4 b, f32x4 acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}

// The same tile product on the bf16 matrix cores (16x16x32 form, 16 cycles,
// against 4 x 32 for the fp32 form), for operands of which AX / BX are exactly
// representable in bf16 (values widened from bf16 inputs).  An operand that is
// not is split as hi + lo, hi = bf16(x), lo = bf16(x - hi), which keeps about 17
// significant bits: one exact operand takes one instruction (slots 0-3 hold hi,
// 4-7 lo, against the exact operand in both halves), two split ones two (the
// lo x lo term, below 2^-16 relative, is dropped).  Products are exact and sums
// fp32, so the result is the fp32 product to about 2^-17 relative.  SPLIT false
// keeps the fp32 form.
__device__ __forceinline__ void split_bf16(f32x4 x, u32x2& hi, u32x2& lo)
{
    hi = pack_bf16x4(x);
    const f32x4 h = {__uint_as_float(hi.x << 16), __uint_as_float(hi.x & 0xffff0000u),
                     __uint_as_float(hi.y << 16), __uint_as_float(hi.y & 0xffff0000u)};
    lo = pack_bf16x4(x - h);
}

template <bool SPLIT, bool AX, bool BX>
__device__ __forceinline__ f32x4 mmt(f32x4 a, f32x4 b, f32x4 acc)
{
    if constexpr (!SPLIT) {
        return mm16(a, b, acc);
    } else if constexpr (AX && BX) {
        return mfma16(pack_bf16x4(a), pack_bf16x4(b), acc);
    } else if constexpr (BX) {
        u32x2 ah, al;
        split_bf16(a, ah, al);
        const u32x2 bb = pack_bf16x4(b);
        return mfma32(u32x4{ah.x, ah.y, al.x, al.y}, u32x4{bb.x, bb.y, bb.x, bb.y}, acc);
    } else if constexpr (AX) {
        u32x2 bh, bl;
        split_bf16(b, bh, bl);
        const u32x2 aa = pack_bf16x4(a);
        return mfma32(u32x4{aa.x, aa.y, aa.x, aa.y}, u32x4{bh.x, bh.y, bl.x, bl.y}, acc);
    } else {
        u32x2 ah, al, bh, bl;
        split_bf16(a, ah, al);
        split_bf16(b, bh, bl);
        acc = mfma32(u32x4{ah.x, ah.y, al.x, al.y}, u32x4{bh.x, bh.y, bh.x, bh.y}, acc);
        return mfma16(ah, bl, acc);
    }
}

}  // namespace ttt
