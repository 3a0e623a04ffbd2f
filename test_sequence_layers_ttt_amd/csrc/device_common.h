// Device-side helpers shared by the TTT kernels: bf16 <-> fp32 conversion,
// typed loads/stores of the I/O dtype, raw-word prefetch registers and 16-lane
// row sums.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

// bf16 stored as its raw 16 bits.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u)
{
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename TIO> struct io;

template <> struct io<float> {
    __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};

template <> struct io<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, size_t i)
    {
        return bf16_bits_to_f32(p[i]);
    }
    __device__ __forceinline__ static void store(uint16_t* p, size_t i, float v)
    {
        p[i] = f32_to_bf16_bits(v);
    }
};

// N consecutive elements of the I/O type kept as the raw 32-bit words a load
// returns: widening to fp32 happens only when the words are consumed, so a load
// issued ahead of its use is not waited for at issue (and, as stores share the
// same counter, neither are the stores issued since).
template <typename TIO, int N>
struct RawRow {
    static constexpr int BYTES = N * (int)sizeof(TIO);
    static constexpr int WORDS = BYTES >= 4 ? BYTES / 4 : 1;
    uint32_t w[WORDS];

    __device__ __forceinline__ void load(const TIO* p)
    {
        if constexpr (BYTES % 16 == 0) {
#pragma unroll
            for (int i = 0; i < WORDS; i += 4) {
                const uint4 v = reinterpret_cast<const uint4*>(p)[i / 4];
                w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
            }
        } else if constexpr (BYTES == 8) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            w[0] = v.x; w[1] = v.y;
        } else if constexpr (BYTES == 4) {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        } else {
            w[0] = *reinterpret_cast<const uint16_t*>(p);   // one bf16, zero-extended
        }
    }
    __device__ __forceinline__ float at(int i) const
    {
        if constexpr (sizeof(TIO) == 4) {
            return __uint_as_float(w[i]);
        } else {
            const uint32_t x = w[i >> 1];
            return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
        }
    }
};

// Sum over the 16 lanes of a DPP row (lanes 16m .. 16m+15); every lane of the row
// receives the same sum, bit for bit (each lane adds the same pairs).  Swaps inside
// each quad (lane ^ 1, lane ^ 2), then the half-row mirror (quad 0 <-> quad 1 of
// each 8-lane half) and the row mirror (half 0 <-> half 1); no cross-row
// movement, no LDS.
__device__ __forceinline__ float dpp_add(float x, int y)
{
    return x + __int_as_float(y);
}

constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float row_sum16(float x)
{
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kDppQuadXor1, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kDppQuadXor2, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kDppRowHalfMirror, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kDppRowMirror, 0xF, 0xF, false));
    return x;
}

// one DPP stage of row_sum16 over N independent values: every move first, then
// every add, so that each move's wait for the previous add is filled by the others
template <int CTRL, int N>
__device__ __forceinline__ void dpp_stage(float (&x)[N])
{
    int m[N];
#pragma unroll
    for (int i = 0; i < N; ++i) m[i] = __builtin_amdgcn_mov_dpp(__float_as_int(x[i]), CTRL, 0xF, 0xF, false);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = dpp_add(x[i], m[i]);
}

// row_sum16 of N independent values (the same sums, stage by stage)
template <int N>
__device__ __forceinline__ void row_sum16_n(float (&x)[N])
{
    dpp_stage<kDppQuadXor1>(x);
    dpp_stage<kDppQuadXor2>(x);
    dpp_stage<kDppRowHalfMirror>(x);
    dpp_stage<kDppRowMirror>(x);
}

}  // namespace ttt
