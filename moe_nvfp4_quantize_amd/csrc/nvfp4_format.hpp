// nvfp4_format.hpp -- NVFP4 element and scale encodings for the gfx950 kernels.
//
// Qwen3.8-Flash-Next-NVFP4 page, section "Core: the W4A4 two-level scaling
// mechanism": elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit; grid
// 0, 0.5, 1, 1.5, 2, 3, 4, 6), block scales are E4M3 (largest value 448, so the
// E4M3FN variant: bias 7, subnormal step 2^-9), the global scale is FP32.
// Rounding is to nearest, ties to even, for both narrow formats.
//
// Everything here is plain float/integer code marked __host__ __device__ so that
// the same functions can be exercised on the CPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define NVFP4_HD __host__ __device__ __forceinline__

namespace nvfp4 {

NVFP4_HD uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
NVFP4_HD float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// 6 (largest E2M1) * 448 (largest E4M3): the global scale is amax / 2688.
constexpr float kGlobalDivisor = 2688.0f;
constexpr float kE4M3Max = 448.0f;

// E4M3FN code of v in [0, 448], round to nearest even.
//  - below 2^-6 the format is uniform with step 2^-9: the code is the number of
//    steps (8 steps is 2^-6, which is code 0x08 as well);
//  - from 2^-6 up, drop 20 of the float's 23 mantissa bits with round to
//    nearest even, then rebias the exponent from 127 to 7.
NVFP4_HD uint32_t e4m3_encode(float v) {
  if (v < 0x1p-6f) return (uint32_t)__builtin_rintf(v * 512.0f);
  uint32_t b = f2u(v);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  uint32_t e = (b >> 23) - 120u;  // - 127 + 7
  uint32_t m = (b >> 20) & 7u;
  return (e << 3) | m;
}

// Value of a positive E4M3FN code (1..126) as float (exact).
NVFP4_HD float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0u) return (float)m * 0x1p-9f;
  return u2f(((e + 120u) << 23) | (m << 20));
}

// E2M1 code of y: nearest grid magnitude of min(|y|, 6), ties to the even code,
// sign bit copied from y (so -0 and negatives that round to 0 give 0x8).
// The grid is uniform by pieces: step 0.5 below 2, step 1 on [2, 4], step 2 on
// [4, 6]; on each piece the code offset is rint of the distance in steps.  Each
// subtraction is exact (Sterbenz), and 2a is exact.
NVFP4_HD uint32_t e2m1_encode(float y) {
  float a = __builtin_fminf(__builtin_fabsf(y), 6.0f);
  uint32_t c;
  if (a < 2.0f)
    c = (uint32_t)__builtin_rintf(2.0f * a);
  else if (a < 4.0f)
    c = 4u + (uint32_t)__builtin_rintf(a - 2.0f);
  else
    c = 6u + (uint32_t)__builtin_rintf((a - 4.0f) * 0.5f);
  return c | ((f2u(y) >> 28) & 8u);
}

// Per-block scale step of the quantizer: returns the E4M3 code and writes the
// encode multiplier r = 1 / (s * g).
//   s32 = bmax / (6 g) ; s = E4M3(min(s32, 448)) ; s = 2^-9 if it rounds to 0.
NVFP4_HD uint32_t block_scale(float bmax, float six_g, float g, float *r) {
  float s32 = __builtin_fminf(bmax / six_g, kE4M3Max);
  uint32_t sc = e4m3_encode(s32);
  if (sc == 0u) sc = 1u;
  *r = 1.0f / (e4m3_value(sc) * g);
  return sc;
}

// bfloat16 <-> float.
NVFP4_HD float bf16_lo(uint32_t w) { return u2f(w << 16); }
NVFP4_HD float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }
NVFP4_HD uint32_t float_to_bf16_bits(float f) {  // round to nearest even, finite f
  uint32_t b = f2u(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace nvfp4
