// Device-side helpers shared by the TTT kernels: bf16 <-> fp32 conversion and
// typed loads/stores of the I/O dtype.
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

}  // namespace ttt
