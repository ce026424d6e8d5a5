// Device helpers for the gfx950 (CDNA4) kernels of libpa: storage formats,
// conversions, wavefront reductions.  Wave size is 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// Running maximum before any key: finite, so exp2(m - m_new) never sees
// (-inf) - (-inf).
constexpr float kNoMax = -3.0e38f;

__host__ __device__ constexpr int dtype_bytes(int dt) {
  return dt == PA_F32 ? 4 : (dt == PA_FP8_E4M3 ? 1 : 2);
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).x;
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w).y;
}

// Two OCP E4M3FN codes (bytes 0,1 or 2,3 of w) -> float32, exact.
__device__ __forceinline__ float2_t fp8x2_lo(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}
__device__ __forceinline__ float2_t fp8x2_hi(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
}

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float32 -> float16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Load element i of a row of dtype dt as float32.
__device__ __forceinline__ float load_as_f32(const void* base, int64_t i, int dt) {
  if (dt == PA_F32) return ((const float*)base)[i];
  uint16_t b = ((const uint16_t*)base)[i];
  if (dt == PA_F16) return (float)__builtin_bit_cast(_Float16, b);
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ void store_from_f32(void* base, int64_t i, int dt, float x) {
  if (dt == PA_F32)
    ((float*)base)[i] = x;
  else if (dt == PA_F16)
    ((uint16_t*)base)[i] = f32_to_f16_bits(x);
  else
    ((uint16_t*)base)[i] = f32_to_bf16_bits(x);
}

// ------------------------------------------------------- fp8 E4M3 storing

// x / s rounded once in float32, then (pack4_fp8) RNE to E4M3FN saturating
// at +-448.  Clamping first is exact: every |x/s| >= 448 rounds to 448 when
// saturating.
__device__ __forceinline__ float fp8_prep(float x, float s) {
  const float y = __fdiv_rn(x, s);
  return __builtin_isnan(y) ? y : fminf(fmaxf(y, -448.f), 448.f);
}

__device__ __forceinline__ uint32_t pack4_fp8(const float* y) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  return (uint32_t)w;
}

// Eight codes requantised from scale s_old to divisor d:
// RNE-saturate((decode(code) * s_old) / d), both steps rounded in float32.
__device__ __forceinline__ uint2 requant8(uint2 w, float s_old, float d) {
  float y[8];
  const float2_t a0 = fp8x2_lo(w.x), a1 = fp8x2_hi(w.x), b0 = fp8x2_lo(w.y), b1 = fp8x2_hi(w.y);
  const float x[8] = {a0.x, a0.y, a1.x, a1.y, b0.x, b0.y, b1.x, b1.y};
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fp8_prep(__fmul_rn(x[i], s_old), d);
  return make_uint2(pack4_fp8(y), pack4_fp8(y + 4));
}

// -------------------------------------------------------------- reductions

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i inside each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of a group ends with the group's sum.  All lanes must be active.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (G >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (G >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (G >= 16) x += dpp<kDppMirror>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  if constexpr (G >= 64) x += __shfl_xor(x, 32);
  return x;
}

}  // namespace pa
