// Shared device helpers for the paged KV-cache kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bit casts
__device__ __forceinline__ float as_float(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------- bfloat16
// Widening keeps the 16 stored bits as the high half of a binary32.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return as_float(pair & 0xFFFF0000u); }

// binary32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- FP8 E4M3
// OCP E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
// is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; largest finite 448.
//
// Encode a binary32 value: round to nearest even, saturate every magnitude
// >= 448 (and infinities) to 448, keep NaN.  Written from the format
// definition with integer rounding so that every code is reproducible.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;           // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;          // |x| >= 448 -> 448
  if (a < 0x3C800000u) {                              // |x| < 2^-6: step 2^-9
    // |x| * 512 is exact (power-of-two scale); rint rounds half to even.
    const uint32_t m = (uint32_t)__builtin_rintf(as_float(a) * 512.0f);
    return sign | m;                                  // m == 8 is 2^-6 = 0x08
  }
  // normal: keep 3 of 23 mantissa bits, round half to even on the dropped 20
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t e = (r >> 23) - 120u;                // rebias 127 -> 7
  uint32_t code = (e << 3) | ((r >> 20) & 7u);
  code = code > 0x7Eu ? 0x7Eu : code;
  return sign | code;
}

// Four binary32 values, none of them NaN, to four codes (byte i holds value
// i), equal to e4m3_encode of each: the clamp to [-448, 448] gives the
// saturation (infinities included), and the hardware conversion rounds to
// nearest even, subnormals included.  Callers send chunks that hold a NaN to
// e4m3_encode instead (a clamp would turn NaN into a finite value).
__device__ __forceinline__ uint32_t e4m3x4_encode_no_nan(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Two codes (kHighWord false: bytes 0,1 of the dword; true: bytes 2,3) to
// two binary32 values, exact (hardware OCP conversion on gfx950).
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <bool kHighWord>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t packed) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)packed, kHighWord);
}

// Two codes to a packed pair of bfloat16, exact (every E4M3 value is a
// bfloat16 value).  Scale 1.0 keeps the conversion a pure re-encoding.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <bool kHighWord>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t packed) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)packed, 1.0f, kHighWord);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- INT4
// 4-bit integer code with zero point 8: the integer nearest to y (ties to
// even) limited to [-8, 7], plus 8; NaN gives 8 (value 0).
__device__ __forceinline__ uint32_t int4_encode(float y) {
  const float k = fminf(fmaxf(__builtin_rintf(y), -8.0f), 7.0f);
  return y == y ? (uint32_t)((int)k + 8) : 8u;
}

// Eight codes (element n in bits 4n .. 4n + 3) packed from eight values
// already multiplied by the inverse scale.
__device__ __forceinline__ uint32_t int4_pack8(const float* y) {
  uint32_t w = 0;
#pragma unroll
  for (int n = 0; n < 8; ++n) w |= int4_encode(y[n]) << (4 * n);
  return w;
}

// ---------------------------------------------------------------- dot products
// a.x*b.x + a.y*b.y + c on packed bfloat16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- lane exchange
// DPP row controls (a row is 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_uint(v), kCtrl, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 1..64, a power of two); every lane
// of a group ends with the group's total.  Groups of <= 16 use DPP.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------------------- misc
// b > 0; a + b - 1 is never formed for a > 0, so no int overflow near INT_MAX
__host__ __device__ __forceinline__ int ceil_div(int a, int b) {
  return a > 0 ? (a - 1) / b + 1 : (a + b - 1) / b;
}

// Bits per element of a cache type (compile-time use in the kernels).
__host__ __device__ constexpr int kv_bits(int dt) {
  return dt == PKV_F32 ? 32 : (dt == PKV_BF16 ? 16 : (dt == PKV_FP8_E4M3 ? 8 : 4));
}

}  // namespace pkv
