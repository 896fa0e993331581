// Device-side helpers shared by the kernels of libsa.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// bf16 -> f32 is exact: the bf16 pattern is the upper half of the f32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return bits_f32(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return bits_f32(pair & 0xffff0000u); }

// f32 -> bf16, round to nearest, ties to even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = f32_bits(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swap a value with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float v) {
    return __shfl_xor(v, 32, kWave);
}

}  // namespace sa
