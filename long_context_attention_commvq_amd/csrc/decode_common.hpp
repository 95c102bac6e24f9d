// Device helpers shared by the decode kernels.
#pragma once

#include <type_traits>
#include <utility>

#include "commvq_internal.hpp"

namespace commvq {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each i a compile-time
// constant (MFMA broadcast selectors must be immediates)
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Phase e^{i m theta_p} of position m from the 64-bit fixed-point turn count
// F_p = theta_p / (2 pi) * 2^64: the top 32 bits of (m * F_p) mod 2^64 are the
// phase in turns, exact to 2^-32 turn for any m < 2^32.
__device__ __forceinline__ float2 phase_exact(uint32_t m, uint32_t flo, uint32_t fhi) {
  const uint32_t turns = m * fhi + __umulhi(m, flo);
  const float x = (float)(int32_t)turns * 0x1p-31f;  // angle / pi in [-1, 1)
  float s, c;
  sincospif(x, &s, &c);
  return make_float2(c, s);
}

// The same phase from the hardware sine and cosine, whose input is in turns
// (measured within 1.2e-7 of the exact values on [0, 1) turn): for values that
// are rounded to fp16, or carried in fp32 for a few steps.
__device__ __forceinline__ float2 phase_hw(uint32_t m, uint32_t flo, uint32_t fhi) {
  const uint32_t turns = m * fhi + __umulhi(m, flo);
  const float x = (float)turns * 0x1p-32f;  // [0, 1) turn
  return make_float2(__builtin_amdgcn_cosf(x), __builtin_amdgcn_sinf(x));
}

// Wavefront reductions: butterfly over the 16 lanes of a row with DPP moves,
// then the four row results combined through scalar lane reads.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4e>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xb1>(v);
  v += dpp_f<0x4e>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace commvq
