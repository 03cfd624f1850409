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
// Both are computed and one is selected, so the GPU runs it without branching.
NVFP4_HD uint32_t e4m3_encode(float v) {
  const uint32_t sub = (uint32_t)__builtin_rintf(v * 512.0f);
  uint32_t b = f2u(v);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t nrm = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);  // exponent - 127 + 7
  return v < 0x1p-6f ? sub : nrm;
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

// fl(a / b), the IEEE quotient, from y = fl(1 / b) with two FMAs: q = fl(a y)
// is within an ulp of a / b, r = a - q b is exact, and fl(q + r y) is the
// correctly rounded quotient (Markstein's theorem, binary floating point with
// a correctly rounded reciprocal; valid while the quotient is a normal float).
NVFP4_HD float div_rn(float a, float b, float y) {
  const float q = a * y;
  const float r = __builtin_fmaf(-q, b, a);
  return __builtin_fmaf(r, y, q);
}

// Block scale code from the block max (quantizer steps 3-4):
//   s32 = bmax / (6 g) ; s = E4M3(min(s32, 448)) ; s = 2^-9 if it rounds to 0.
// six_g = fl(6 g), inv_six_g = fl(1 / six_g).  Quotients below 2^-10 all give
// code 1 and quotients above 448 all give 448, so the division only has to be
// exact in between, where div_rn is.
NVFP4_HD uint32_t block_scale_code(float bmax, float six_g, float inv_six_g) {
  const uint32_t sc = e4m3_encode(__builtin_fminf(div_rn(bmax, six_g, inv_six_g), kE4M3Max));
  return sc ? sc : 1u;
}

// Block scale code and its encode multiplier r = 1 / (s g).
NVFP4_HD uint32_t block_scale(float bmax, float six_g, float g, float *r) {
  const uint32_t sc = block_scale_code(bmax, six_g, 1.0f / six_g);
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
