// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace hum {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x1_t __attribute__((ext_vector_type(1)));
typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  // the gfx950 conversion instruction (v_cvt_pk_bf16_f32): round to nearest
  // even, a NaN stays a (quiet) NaN
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> a packed bf16 pair (a in the low half), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float a, float b) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// E8M0 code -> float 2^(c-127); 255 -> NaN.  Branch free: code 0 is the
// subnormal 2^-127 (mantissa bit 22 alone), code 255 the quiet NaN
// (all-ones exponent and mantissa bit 22).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  const uint32_t edge = (((c + 1u) & 0xFFu) <= 1u) ? 0x00400000u : 0u;
  return __uint_as_float((c << 23) | edge);
}

// Two floats -> two E4M3 codes (RNE, saturated to +-448, signed zero kept).
// The hardware conversion rounds to nearest even; the clamp makes it
// saturate instead of producing NaN above 448.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// One float -> E2M1 code (nearest, ties to the even code, saturated to +-6,
// sign bit kept for values that round to zero): a comparison against the
// midpoints of the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = __builtin_fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u
                     : a < 0.75f ? 1u
                     : a <= 1.25f ? 2u
                     : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u
                     : a < 3.5f ? 5u
                     : a <= 5.0f ? 6u
                     : 7u;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Sum / max over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane
// of the row receives the result.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false)));
  return v;
}

// Max over the 4 lanes of a DPP quad.
__device__ __forceinline__ float quad_max(float v) {
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
  return v;
}

// floor(log2(a)) for a finite float a > 0, from the exponent field.
__device__ __forceinline__ int floor_log2_f32(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF);
  if (e == 0) return 31 - __builtin_clz(u & 0x007FFFFFu) - 149;  // subnormal
  return e - 127;
}

// MX scale exponent code for a block whose absolute maximum is `amax`, for
// elements whose largest power of two is 2^emax (E4M3: 8, E2M1: 2).
__device__ __forceinline__ int mx_scale_code_emax(float amax, int emax) {
  if (!(amax > 0.0f)) return 127;
  int e = floor_log2_f32(amax) - emax + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}
__device__ __forceinline__ int mx_scale_code(float amax) { return mx_scale_code_emax(amax, 8); }

// 2^(127 - e) as an exact float for e in [0, 254] (the reciprocal of the
// MX block scale 2^(e-127)).
__device__ __forceinline__ float mx_inv_scale(int e) {
  int p = 127 - e;  // -127 .. 127
  if (p >= -126) return __uint_as_float((uint32_t)(p + 127) << 23);
  return __uint_as_float(0x00400000u);  // 2^-127
}

}  // namespace hum
