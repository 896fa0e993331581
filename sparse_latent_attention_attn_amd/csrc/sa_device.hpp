// Device-side helpers shared by the kernels of libsa.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two f32 -> two bf16 in one word (lo in bits 0..15), round to nearest even: gfx950 has a
// packed conversion instruction (v_cvt_pk_bf16_f32) for this.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane exchanges without the LDS pipe (gfx950 permlane swaps). With both operands
// equal, v_permlane32_swap leaves each lane holding its own value and that of lane l ^ 32
// (one in each result), and v_permlane16_swap does the same for lane l ^ 16.
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(f32_bits(v), f32_bits(v), false, false);
    return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(f32_bits(v), f32_bits(v), false, false);
    return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(f32_bits(v), f32_bits(v), false, false);
    return bits_f32(r[0]) + bits_f32(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(f32_bits(v), f32_bits(v), false, false);
    return bits_f32(r[0]) + bits_f32(r[1]);
}

}  // namespace sa
