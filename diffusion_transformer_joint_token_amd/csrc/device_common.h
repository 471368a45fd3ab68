// Device-side helpers shared by the gfx950 kernels of the attention step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even, in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Exchange a value with the lane 32 positions away (lane l <-> l ^ 32) and
// return that partner's value.  permlane32_swap(x, x) yields, per lane, the
// pair {x[l mod 32], x[l mod 32 + 32]}.
__device__ __forceinline__ float partner32(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t lo = r[0], hi = r[1];
  uint32_t mine_is_low = (__lane_id() < 32);
  return __builtin_bit_cast(float, mine_is_low ? hi : lo);
}

__device__ __forceinline__ float max_with_partner32(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float sum_with_partner32(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// sin and cos of a rotary phase given in turns (t = phase / (2 pi)).  The
// whole turns are removed in double (t - rint(t), exact) and the fraction f,
// |f| <= 1/2, rounded once to fp32 (error <= 2^-25 turns); the hardware
// v_sin_f32 / v_cos_f32 take their argument in turns.  Measured on gfx950
// over 2^24 points of [-1/2, 1/2]: absolute error <= 1.3e-7 against double
// precision, as small as an fp32 sincosf after a double-precision reduction,
// for two instructions instead of a library call per pair.
__device__ __forceinline__ void sincos_turns(double t, float& s, float& c) {
  const float f = (float)(t - rint(t));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

}  // namespace dit
