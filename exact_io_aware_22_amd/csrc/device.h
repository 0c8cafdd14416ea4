// Device-side helpers shared by the gfx950 kernels: vector types, bf16 packing,
// base-2 exponentials and cross-lane reductions on 64-wide wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kInfB = __builtin_inff();

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }
// A dword as two bfloat16. Always bit-cast a named value: applied directly to a
// vector-element expression (v[i]) the cast has been seen to read element 0.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2_t, x); }

// Two floats -> two bfloat16 (round to nearest even) in one dword, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// bfloat16 halves of a dword -> float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Combine a per-lane value with the same lane of the other 32-lane half.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace fa
