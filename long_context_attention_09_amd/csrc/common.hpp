// Device helpers shared by the gfx950 kernels: storage codecs, RoPE angles,
// wave reductions and MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) short i16x8;

constexpr float kLog2e = 1.4426950408889634f;

// 2^x on the hardware exp2 unit (one instruction).  Results below 2^-126
// flush to zero; every caller passes x <= 0 for softmax weights relative to a
// running maximum, where such weights are negligible.  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ BF16

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

__device__ __forceinline__ __bf16 u16_as_bf16(uint16_t u) { return __builtin_bit_cast(__bf16, u); }

// Two floats as BF16 (nearest even) in one packed conversion: lo in bits
// 0-15, hi in bits 16-31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Two 4 x 16-bit transposing LDS reads as one BF16 x 8 operand (a first).
__device__ __forceinline__ bf16x8 bf16x8_of(const i16x4& a, const i16x4& b) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------------------ FP8 E4M3FN

// Decode one byte exactly (OCP E4M3FN: bias 7, no inf, S.1111.111 = NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 0) v = (float)m * 0.001953125f;  // m/8 * 2^-6
  else if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return s ? -v : v;
}

// Round-to-nearest-even fp32 -> E4M3FN, saturating at +-448; keeps the sign of
// values that round to zero.  Scaling by powers of two is exact, so rintf
// (round-half-even) on the scaled value gives the correctly rounded code.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (a != a) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid step 2^-9
    const uint32_t q = (uint32_t)rintf(a * 512.0f);  // 0 .. 8 (8 = min normal)
    return sign | q;
  }
  int e;
  const float fr = frexpf(a, &e);            // a = fr * 2^e, fr in [0.5, 1)
  int E = e - 1;                              // a = (2 fr) * 2^E, 2fr in [1, 2)
  uint32_t mant = (uint32_t)rintf((2.0f * fr - 1.0f) * 8.0f);
  if (mant == 8) { mant = 0; ++E; }
  uint32_t code = ((uint32_t)(E + 7) << 3) | mant;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// ------------------------------------------------------------------ MXFP4

// E2M1 code n (sign in bit 3): twice the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
// 6 are the nibbles of 0xC8643210, so the decode needs no table in memory
__device__ __forceinline__ float e2m1_to_f32(uint32_t n) {
  const float v = 0.5f * (float)((0xC8643210u >> (4u * (n & 7u))) & 15u);
  return (n & 8u) ? -v : v;
}

// Shared block exponent floor(log2(amax)) - 2 clamped to [-127, 127]; zero -> -127.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  frexpf(amax, &e);
  int E = (e - 1) - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Nearest E2M1 code of |v| with ties to the even code, clamped to 6; the
// thresholds are the midpoints of the grid {0, .5, 1, 1.5, 2, 3, 4, 6}
// (a tie goes to the neighbour with an even code).
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float v = fabsf(x);
  uint32_t c = (v > 0.25f) + (v >= 0.75f) + (v > 1.25f) + (v >= 1.75f) + (v > 2.5f) +
               (v >= 3.5f) + (v > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// ------------------------------------------------------------------ RoPE

// cos / sin of pos * theta^(-2u/d_rope): the angle is formed and reduced to
// one turn in fp64 (at positions near 2^20 an fp32 angle would be off by
// ~0.06 rad); sin and cos of the reduced angle are taken in fp32.
__device__ __forceinline__ void rope_cos_sin(double pos, int u, int d_rope, double log_theta,
                                             float* c, float* s) {
  const double inv_freq = exp(-2.0 * (double)u / (double)d_rope * log_theta);
  double ang = pos * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  ang = ang - two_pi * floor(ang * (1.0 / two_pi));
  sincosf((float)ang, s, c);
}

// ------------------------------------------------------------------ wave helpers

// Cross-lane move within rows of 16 lanes (DPP control CTRL: quad_perm,
// row_half_mirror or row_mirror), no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes, the same value in every lane: DPP within each row of
// 16 (lane ^ 1, lane ^ 2, mirrored half rows, mirrored rows), then the four
// row sums through readlane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// fp32 score -> uint32 whose unsigned order is the float order.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t x = __float_as_uint(f);
  return x ^ ((uint32_t)((int32_t)x >> 31) | 0x80000000u);   // ~x when negative, x | 2^31 otherwise
}

}  // namespace csa
