// quantize.hip -- dynamic / static two-level NVFP4 quantization on gfx950,
// and the kernels' other modes on the same data path: four-over-six block
// scales, quantize-dequantize, and FP8 E4M3 per-tensor quantization.
//
// Qwen3.8-Flash-Next-NVFP4 page, section "Core: the W4A4 two-level scaling
// mechanism" (level 1: one E4M3 scale per 16 elements along the last dimension;
// level 2: one FP32 scale per tensor) and sub-section "The A4 side: dynamic
// activations" (activations quantized on the fly with the same rule).
//
// Every kernel walks x in units of 16 consecutive elements of a row and takes a
// mode (enum Mode) that decides what a unit becomes; the per-mode encoders sit
// next to the plain one below.
//
// The dynamic global scale needs max|x| over the whole tensor before any block
// can be encoded.  Two kernels implement that:
//
//  * resident (one HBM read): one workgroup per CU, 1024 threads (four waves
//    per SIMD, up to 10 bf16 / 4 fp32 blocks per thread in 128 VGPRs) or 512
//    threads (two waves per SIMD, up to 20 bf16 / 10 fp32 blocks in 256
//    VGPRs).  Every thread loads its U 16-element blocks into registers and
//    keeps their block maxima; each workgroup publishes its max and waits for
//    all others', then every thread encodes its blocks from registers.  Used
//    when the tensor fits in the register file (up to about 42 M bf16 or 21 M
//    fp32 elements on 256 CUs).
//  * two-pass (fallback for larger tensors, and the batched per-matrix form):
//    an amax pass writes one partial per workgroup; the encode pass reduces the
//    partials and re-reads x.
//
// Encoding one block (all float32, round to nearest even; the order of the
// float32 steps is part of the specification and must not be fused):
//    s = E4M3(min(bmax / (6 g), 448)), 2^-9 if that rounds to 0   [software;
//                                      the quotient by div_rn, bit-identical
//                                      to the IEEE division]
//    r = 1 / (s g)                     [per-workgroup table over the 126 codes]
//    y = x * r ;  code = E2M1(y)       [hardware v_cvt_scalef32_pk_fp4_f32 with
//                                       unit scale: round to nearest even,
//                                       saturating at 6, sign kept on zero]
// A thread owns whole blocks, so the block max needs no cross-lane traffic;
// consecutive threads own consecutive blocks, so a wave reads 2 KB (bf16) or
// 4 KB (fp32) of contiguous input and writes 512 B of codes and 64 B of scales.
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"

#include <algorithm>

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;          // two-pass kernels
constexpr uint32_t kSpinLimit = 1u << 15;  // arrival wait bound (tens of milliseconds)

// What a launch writes for each 16-element unit of x.
enum Mode : int {
  kNvfp4 = 0,  // packed E2M1 codes + E4M3 block scale
  kFour6 = 1,  // the same, block scale by the four-over-six rule
  kQdq = 2,    // the decoded values, in the input type (quantize-dequantize)
  kFp8 = 3,    // 16 E4M3 codes, one per element, per-tensor scale only
};

// 16 consecutive elements starting at p, as raw words (bf16: 8 dwords holding
// two values each; fp32: 16 dwords).  VEC: p is 16-byte aligned.
template <typename T>
struct Raw;
template <>
struct Raw<uint16_t> {
  static constexpr int W = 8;
};
template <>
struct Raw<float> {
  static constexpr int W = 16;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// STREAM: the data is read once by this launch; non-temporal loads keep it
// from being allocated on its way through the caches, which on MI355X takes
// a cold read of the tensor from about 3.3 to about 6.2 TB/s.  The first pass
// of the two-pass path reads with normal loads so that the second may still
// find part of the tensor in the Infinity Cache.
template <typename T, bool VEC, bool STREAM = true>
__device__ __forceinline__ void load_raw(const T *p, uint32_t w[Raw<T>::W]) {
  if (VEC) {
    const u32x4 *p4 = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < Raw<T>::W / 4; ++i) {
      const u32x4 t = STREAM ? __builtin_nontemporal_load(p4 + i) : p4[i];
      w[4 * i] = t[0];
      w[4 * i + 1] = t[1];
      w[4 * i + 2] = t[2];
      w[4 * i + 3] = t[3];
    }
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = f2u(p[i]);
  }
}

template <typename T>
__device__ __forceinline__ float elem(const uint32_t w[Raw<T>::W], int i) {
  if constexpr (sizeof(T) == 2) return (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
  else return u2f(w[i]);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// max |x| of a block.  bf16: on the packed bits (|x| is the low 15 bits of each
// half, and non-negative floats order like their bit patterns), so the floats
// need not be kept in registers until the encode.
template <typename T>
__device__ __forceinline__ float raw_max(const uint32_t w[Raw<T>::W]) {
  if constexpr (sizeof(T) == 2) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return u2f((uint32_t)(m2[0] > m2[1] ? m2[0] : m2[1]) << 16);
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) m = fmaxf(m, fmaxf(fabsf(elem<T>(w, i)), fabsf(elem<T>(w, i + 1))));
    return m;
  }
}

// Encode one block: scale code from the block max, 16 codes from x * r.  The
// outputs are written once and not read back by this kernel: non-temporal
// stores keep them from lingering dirty in L2.
template <typename T>
__device__ __forceinline__ void encode_block(const uint32_t w[Raw<T>::W], float bmax, float six_g,
                                             float inv_six_g, const float *rtab, uint8_t *q,
                                             uint8_t *s) {
  const uint32_t sc = block_scale_code(bmax, six_g, inv_six_g);
  const float r = rtab[sc];
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 0) * r, elem<T>(w, 1) * r, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 2) * r, elem<T>(w, 3) * r, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 4) * r, elem<T>(w, 5) * r, 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 6) * r, elem<T>(w, 7) * r, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 8) * r, elem<T>(w, 9) * r, 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 10) * r, elem<T>(w, 11) * r, 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 12) * r, elem<T>(w, 13) * r, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 14) * r, elem<T>(w, 15) * r, 1.0f, 3);
  __builtin_nontemporal_store((uint64_t)lo | ((uint64_t)hi << 32), reinterpret_cast<uint64_t *>(q));
  __builtin_nontemporal_store((uint8_t)sc, s);
}

// 16 E2M1 codes of x * r as two dwords (element 2i in the low nibble of byte i)
template <typename T>
__device__ __forceinline__ uint64_t encode16(const uint32_t w[Raw<T>::W], float r) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 0) * r, elem<T>(w, 1) * r, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 2) * r, elem<T>(w, 3) * r, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 4) * r, elem<T>(w, 5) * r, 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, elem<T>(w, 6) * r, elem<T>(w, 7) * r, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 8) * r, elem<T>(w, 9) * r, 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 10) * r, elem<T>(w, 11) * r, 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 12) * r, elem<T>(w, 13) * r, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, elem<T>(w, 14) * r, elem<T>(w, 15) * r, 1.0f, 3);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

typedef float float2v __attribute__((ext_vector_type(2)));

// Sum of squared errors of a block's 16 decoded values against x, in float32
// and in element order: d = x - fl(v * g) with v = e2m1(code) * s exact.
template <typename T>
__device__ __forceinline__ float block_sse(const uint32_t w[Raw<T>::W], uint64_t codes, float sv,
                                           float g) {
  float e = 0.0f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t c = (uint32_t)(codes >> (32 * half));
    float2v v[4];
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xh = (v[i / 2][i % 2] * sv) * g;
      const float d = elem<T>(w, 8 * half + i) - xh;
      e = e + d * d;
    }
  }
  return e;
}

// Four-over-six encode of one block: the block max mapped to E2M1 magnitude 6
// (plain) or 4, whichever has the lower float32 squared error (ties: 6).
// Nemotron 3.5 Lightning QAD page, PTQ recipe table ("4/6").
template <typename T>
__device__ __forceinline__ void encode_block_4over6(const uint32_t w[Raw<T>::W], float bmax, float g,
                                                    float six_g, float inv_six_g, float four_g,
                                                    float inv_four_g, const float *rtab, uint8_t *q,
                                                    uint8_t *s) {
  const uint32_t sc6 = block_scale_code(bmax, six_g, inv_six_g);
  const uint32_t sc4 = block_scale_code(bmax, four_g, inv_four_g);
  const uint64_t c6 = encode16<T>(w, rtab[sc6]);
  const uint64_t c4 = encode16<T>(w, rtab[sc4]);
  const float e6 = block_sse<T>(w, c6, e4m3_value(sc6), g);
  const float e4 = block_sse<T>(w, c4, e4m3_value(sc4), g);
  const bool take4 = e4 < e6;
  __builtin_nontemporal_store(take4 ? c4 : c6, reinterpret_cast<uint64_t *>(q));
  __builtin_nontemporal_store((uint8_t)(take4 ? sc4 : sc6), s);
}

// Quantize-dequantize of one block: the plain encode, then every value decoded
// back, fl32(e2m1 * s * g) (e2m1 * s exact), written in T (bf16: rounded to
// nearest even).  QAD page: the simulated-quantization forward.
template <typename T, bool VEC>
__device__ __forceinline__ void qdq_block(const uint32_t w[Raw<T>::W], float bmax, float six_g,
                                          float inv_six_g, const float *rtab, float g, T *y) {
  const uint32_t sc = block_scale_code(bmax, six_g, inv_six_g);
  const uint64_t codes = encode16<T>(w, rtab[sc]);
  const float sv = e4m3_value(sc);
  float o[16];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t c = (uint32_t)(codes >> (32 * half));
    float2v v[4];
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[8 * half + i] = (v[i / 2][i % 2] * sv) * g;
  }
  if constexpr (sizeof(T) == 2) {
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pk[i] = float_to_bf16_bits(o[2 * i]) | (float_to_bf16_bits(o[2 * i + 1]) << 16);
    if (VEC) {
      u32x4 *y4 = reinterpret_cast<u32x4 *>(y);
      __builtin_nontemporal_store((u32x4){pk[0], pk[1], pk[2], pk[3]}, y4);
      __builtin_nontemporal_store((u32x4){pk[4], pk[5], pk[6], pk[7]}, y4 + 1);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = (T)(pk[i / 2] >> (16 * (i % 2)));
    }
  } else {
    if (VEC) {
      u32x4 *y4 = reinterpret_cast<u32x4 *>(y);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_nontemporal_store((u32x4){f2u(o[4 * k]), f2u(o[4 * k + 1]), f2u(o[4 * k + 2]),
                                            f2u(o[4 * k + 3])}, y4 + k);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = o[i];
    }
  }
}

// FP8 W8A8 (per-tensor E4M3) encode of one 16-element unit: y = x * r with
// r = 1 / g, clamped to [-448, 448] (a static scale below the data's range
// saturates instead of producing the NaN code), then the hardware
// float32 -> E4M3FN convert, two values per instruction, round to nearest
// even, sign kept on zero.  QAD tutorial, table of quantized tensors (the
// attention projections stay FP8 W8A8); format-selection guide, section 1
// (FP8 W8A8 with per-tensor scaling).
template <typename T>
__device__ __forceinline__ void encode_unit_fp8(const uint32_t w[Raw<T>::W], float r, uint8_t *q) {
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_fmed3f(elem<T>(w, 4 * k + e) * r, -448.0f, 448.0f);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);
    o[k] = (uint32_t)v;
  }
  __builtin_nontemporal_store((u32x4){o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4 *>(q));
}

// r = 1 / (s * g) for every positive E4M3 code s (index 1..126); one per thread.
__device__ __forceinline__ void fill_rtab(float *rtab, float g) {
  const uint32_t c = threadIdx.x;
  if (c < 128) rtab[c] = (c >= 1u && c <= 126u) ? 1.0f / (e4m3_value(c) * g) : 0.0f;
}

// Per-tensor decode scale from the tensor's max |x|: amax / (6 * 448) for
// NVFP4 (the block holding amax gets block scale 448), amax / 448 for FP8 (the
// largest element gets the largest code); 1 for an all-zero tensor.
template <int MODE>
__device__ __forceinline__ float global_from_amax(float amax) {
  return amax > 0.0f ? amax / (MODE == kFp8 ? kE4M3Max : kGlobalDivisor) : 1.0f;
}

// ------------------------------------------------------------ two-pass path

// One workgroup per partial (at most 256 per matrix, so as few as one per CU):
// each thread keeps NU blocks (256 bytes) of loads in flight per iteration.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(QuantParams p) {
  constexpr uint32_t NU = 256 / (16 * sizeof(T));
  const uint32_t b = blockIdx.y;
  const T *x = static_cast<const T *>(p.x) + (int64_t)b * p.x_mstride;
  const uint32_t stride = gridDim.x * kThreads;
  auto at = [&](uint32_t u) {
    const uint32_t row = p.div_nbpr.div(u);
    return x + (int64_t)row * p.ld + (u - row * p.nbpr) * 16;
  };
  float m = 0.0f;
  uint32_t u = blockIdx.x * kThreads + threadIdx.x;
  for (; (uint64_t)u + (NU - 1) * (uint64_t)stride < p.units; u += NU * stride) {
    uint32_t w[NU][Raw<T>::W];
#pragma unroll
    for (uint32_t i = 0; i < NU; ++i) load_raw<T, VEC, false>(at(u + i * stride), w[i]);
#pragma unroll
    for (uint32_t i = 0; i < NU; ++i) m = fmaxf(m, raw_max<T>(w[i]));
  }
  for (; u < p.units; u += stride) {
    uint32_t w[Raw<T>::W];
    load_raw<T, VEC, false>(at(u), w);
    m = fmaxf(m, raw_max<T>(w));
  }
  m = block_max(m);
  if (threadIdx.x == 0) p.partials[(int64_t)b * p.P + blockIdx.x] = m;
}

template <typename T, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  __shared__ float rtab[128];
  const uint32_t b = blockIdx.y;
  float g;
  if (p.static_global) {
    g = p.g[b];
  } else {
    float m = 0.0f;
    for (uint32_t i = threadIdx.x; i < p.P; i += kThreads) m = fmaxf(m, p.partials[(int64_t)b * p.P + i]);
    m = block_max(m);
    g = global_from_amax<MODE>(m);
    if (blockIdx.x == 0 && threadIdx.x == 0) p.g[b] = g;
  }
  if (MODE != kFp8) fill_rtab(rtab, g);
  __syncthreads();
  const float six_g = 6.0f * g, inv_six_g = 1.0f / six_g, r8 = 1.0f / g;
  const T *x = static_cast<const T *>(p.x) + (int64_t)b * p.x_mstride;
  uint8_t *q = p.q + (int64_t)b * p.q_mstride;
  uint8_t *s = p.s + (int64_t)b * p.s_mstride;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < p.units; u += gridDim.x * kThreads) {
    const uint32_t row = p.div_nbpr.div(u);
    const uint32_t blk = u - row * p.nbpr;
    uint32_t w[Raw<T>::W];
    load_raw<T, VEC>(x + (int64_t)row * p.ld + blk * 16, w);
    // u == row * nbpr + blk and q/s rows are dense: offsets are u*8 and u
    // (FP8: u*16)
    if (MODE == kFp8)
      encode_unit_fp8<T>(w, r8, q + (int64_t)u * 16);
    else if (MODE == kQdq)
      qdq_block<T, VEC>(w, raw_max<T>(w), six_g, inv_six_g, rtab, g,
                        static_cast<T *>(p.y) + (int64_t)row * p.ld_y + blk * 16);
    else if (MODE == kFour6)
      encode_block_4over6<T>(w, raw_max<T>(w), g, six_g, inv_six_g, 4.0f * g, 1.0f / (4.0f * g), rtab,
                             q + (int64_t)u * 8, s + u);
    else
      encode_block<T>(w, raw_max<T>(w), six_g, inv_six_g, rtab, q + (int64_t)u * 8, s + u);
  }
}

// ------------------------------------------------------------ resident path

// Max |x| over the whole tensor read by one workgroup alone: the way out when
// the other workgroups of a launch do not all become resident in time.
template <typename T, bool VEC>
__device__ float whole_tensor_max(const QuantParams &p) {
  const T *x = static_cast<const T *>(p.x);
  float m = 0.0f;
  for (uint32_t u = threadIdx.x; u < p.units; u += blockDim.x) {
    const uint32_t row = p.div_nbpr.div(u);
    uint32_t w[Raw<T>::W];
    load_raw<T, VEC>(x + (int64_t)row * p.ld + (u - row * p.nbpr) * 16, w);
    m = fmaxf(m, raw_max<T>(w));
  }
  return block_max(m);
}

// Single HBM read.  Cross-workgroup traffic is relaxed atomics on single words
// only (no release/acquire fences, which on a multi-XCD GPU write back and
// invalidate L2): workgroup w publishes 0x80000000 | bits(its max) into
// slot[parity][w] and waits until slots 0..G-1 all carry the flag.  The other
// parity's slots are cleared for the next launch, and the last workgroup to
// finish flips the parity.  A wait that runs past its bound (workgroups not
// co-resident) is not an error: that workgroup reads the whole tensor itself,
// which yields the same max.
template <typename T, bool VEC, int U, int NT, int MODE>
__global__ __launch_bounds__(NT) void resident_kernel(QuantParams p, ResidentState *st) {
  __shared__ float rtab[128];
  __shared__ uint32_t s_fallback, s_lim;
  const uint32_t tid = threadIdx.x, G = gridDim.x;
  const uint32_t stride = G * NT;
  const T *x = static_cast<const T *>(p.x);
  const uint32_t par = __hip_atomic_load(&st->parity, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u;
  for (uint32_t i = blockIdx.x * NT + tid; i < kMaxResidentWGs; i += stride)
    __hip_atomic_store(&st->slot[par ^ 1u][i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // phase 1: every block of this thread into registers, with its max
  uint32_t w[U][Raw<T>::W];
  float bmax[U];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const uint32_t u = i * stride + blockIdx.x * NT + tid;
    if (u < p.units) {
      const uint32_t row = p.div_nbpr.div(u);
      load_raw<T, VEC>(x + (int64_t)row * p.ld + (u - row * p.nbpr) * 16, w[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const uint32_t u = i * stride + blockIdx.x * NT + tid;
    const float b = u < p.units ? raw_max<T>(w[i]) : 0.0f;
    if (MODE != kFp8) bmax[i] = b;  // FP8 needs only the tensor's max: no registers kept
    m = fmaxf(m, b);
  }
  m = block_max(m);

  // publish, then gather every workgroup's max
  if (tid == 0) {
    s_fallback = 0u;
    const uint32_t l = __hip_atomic_load(&st->spin_limit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_lim = l ? l : kSpinLimit;
    __hip_atomic_store(&st->slot[par][blockIdx.x], 0x80000000u | f2u(m), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  // the wait bound, read once per workgroup (an agent-scope load of one word by
  // every thread cost a single-read quantize-dequantize pass 30% of its time)
  const uint32_t lim = s_lim;
  float a = 0.0f;
  for (uint32_t i = tid; i < G; i += NT) {
    uint32_t v = 0;
    for (uint32_t spin = 0;; ++spin) {
      v = __hip_atomic_load(&st->slot[par][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v & 0x80000000u) break;
      if (spin >= lim) {
        s_fallback = 1u;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    a = fmaxf(a, u2f(v & 0x7FFFFFFFu));
  }
  a = block_max(a);  // contains a barrier: s_fallback is settled
  if (s_fallback) {
    a = whole_tensor_max<T, VEC>(p);
    if (tid == 0) __hip_atomic_fetch_add(&st->fallbacks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const float g = global_from_amax<MODE>(a);
  if (blockIdx.x == 0 && tid == 0) p.g[0] = g;
  if (MODE != kFp8) fill_rtab(rtab, g);
  __syncthreads();
  const float six_g = 6.0f * g, inv_six_g = 1.0f / six_g, r8 = 1.0f / g;

  // phase 2: encode from registers
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const uint32_t u = i * stride + blockIdx.x * NT + tid;
    if (u < p.units) {
      if (MODE == kFp8) {
        encode_unit_fp8<T>(w[i], r8, p.q + (int64_t)u * 16);
      } else if (MODE == kQdq) {
        const uint32_t row = p.div_nbpr.div(u);
        qdq_block<T, VEC>(w[i], bmax[i], six_g, inv_six_g, rtab, g,
                          static_cast<T *>(p.y) + (int64_t)row * p.ld_y + (u - row * p.nbpr) * 16);
      } else {
        encode_block<T>(w[i], bmax[i], six_g, inv_six_g, rtab, p.q + (int64_t)u * 8, p.s + u);
      }
    }
  }

  // the last workgroup out hands the other slot array to the next launch
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&st->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1) {
      __hip_atomic_store(&st->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&st->parity, par ^ 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename T, bool VEC, int MODE>
hipError_t launch_two_pass(const QuantParams &p, uint32_t batch, hipStream_t stream) {
  uint64_t wg = ((uint64_t)p.units + kThreads - 1) / kThreads;
  if (wg < 1) wg = 1;
  const uint32_t qgrid = (uint32_t)(wg < 2048 ? wg : 2048);
  if (!p.static_global) {
    amax_partials_kernel<T, VEC><<<dim3(p.P, batch), kThreads, 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  quantize_kernel<T, VEC, MODE><<<dim3(qgrid, batch), kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

// Resident workgroups a launch may count on: one per CU.
uint32_t resident_capacity_wgs() { return device_cu_count(); }

template <typename T, bool VEC, int U, int NT, int MODE>
hipError_t launch_resident_u(const QuantParams &p, ResidentState *st, uint32_t G, hipStream_t stream) {
  resident_kernel<T, VEC, U, NT, MODE><<<G, NT, 0, stream>>>(p, st);
  return hipGetLastError();
}

// Blocks per thread U and workgroup size NT: 1024 threads (four waves per
// SIMD, at most 128 VGPRs) while U stays small, 512 threads (256 VGPRs) for
// the largest tensors.  Returns hipErrorInvalidValue when no variant fits.
template <typename T, bool VEC, int MODE>
hipError_t launch_resident(const QuantParams &p, ResidentState *st, uint32_t G, hipStream_t stream) {
  const uint64_t n = p.units;
  auto need = [&](uint64_t nt) { return (n + (uint64_t)G * nt - 1) / ((uint64_t)G * nt); };
  const uint64_t u1024 = need(1024), u512 = need(512);
  if constexpr (sizeof(T) == 2) {
    if (u1024 <= 1) return launch_resident_u<T, VEC, 1, 1024, MODE>(p, st, G, stream);
    if (u1024 <= 2) return launch_resident_u<T, VEC, 2, 1024, MODE>(p, st, G, stream);
    if (u1024 <= 4) return launch_resident_u<T, VEC, 4, 1024, MODE>(p, st, G, stream);
    if (u1024 <= 6) return launch_resident_u<T, VEC, 6, 1024, MODE>(p, st, G, stream);
    if (u1024 <= 8) return launch_resident_u<T, VEC, 8, 1024, MODE>(p, st, G, stream);
    // at 10 blocks per thread the encodes of quantize-dequantize (decode and
    // store) and of FP8 (sixteen converts per block) need more than 128 VGPRs
    if constexpr (MODE == kNvfp4)
      if (u1024 <= 10) return launch_resident_u<T, VEC, 10, 1024, MODE>(p, st, G, stream);
    if (u512 <= 16) return launch_resident_u<T, VEC, 16, 512, MODE>(p, st, G, stream);
    if (u512 <= 20) return launch_resident_u<T, VEC, 20, 512, MODE>(p, st, G, stream);
  } else {
    if (u1024 <= 1) return launch_resident_u<T, VEC, 1, 1024, MODE>(p, st, G, stream);
    if (u1024 <= 2) return launch_resident_u<T, VEC, 2, 1024, MODE>(p, st, G, stream);
    if (u1024 <= 4) return launch_resident_u<T, VEC, 4, 1024, MODE>(p, st, G, stream);
    if (u512 <= 6) return launch_resident_u<T, VEC, 6, 512, MODE>(p, st, G, stream);
    if (u512 <= 8) return launch_resident_u<T, VEC, 8, 512, MODE>(p, st, G, stream);
    if (u512 <= 10) return launch_resident_u<T, VEC, 10, 512, MODE>(p, st, G, stream);
  }
  return hipErrorInvalidValue;
}

// true when launch_resident has a variant for this many blocks on G workgroups
bool resident_fits(uint64_t units, uint32_t G, bool bf16) {
  const uint64_t cap = (uint64_t)G * 512 * (bf16 ? 20 : 10);
  return units <= cap;
}

}  // namespace

uint32_t quantize_partials_per_matrix(uint64_t units) {
  uint64_t wg = (units + kThreads - 1) / kThreads;
  if (wg < 1) wg = 1;
  return (uint32_t)(wg < kMaxPartials ? wg : kMaxPartials);
}

namespace {

template <int MODE>
hipError_t dispatch_two_pass(const QuantParams &p, bool bf16, bool vec, uint32_t batch, hipStream_t stream) {
  if (bf16)
    return vec ? launch_two_pass<uint16_t, true, MODE>(p, batch, stream)
               : launch_two_pass<uint16_t, false, MODE>(p, batch, stream);
  return vec ? launch_two_pass<float, true, MODE>(p, batch, stream)
             : launch_two_pass<float, false, MODE>(p, batch, stream);
}

template <int MODE>
hipError_t dispatch_resident(const QuantParams &p, bool bf16, bool vec, ResidentState *st, uint32_t G,
                             hipStream_t stream) {
  if (bf16)
    return vec ? launch_resident<uint16_t, true, MODE>(p, st, G, stream)
               : launch_resident<uint16_t, false, MODE>(p, st, G, stream);
  return vec ? launch_resident<float, true, MODE>(p, st, G, stream)
             : launch_resident<float, false, MODE>(p, st, G, stream);
}

template <int MODE>
hipError_t dispatch(const QuantParams &p, bool bf16, bool vec, uint32_t batch, ResidentState *st,
                    hipStream_t stream) {
  // single-read resident path: dynamic scale, one matrix, fits in registers
  if (MODE != kFour6 && !p.static_global && batch == 1 && st != nullptr) {
    const uint32_t cus = resident_capacity_wgs();
    uint32_t G = (uint32_t)std::min<uint64_t>(((uint64_t)p.units + 511) / 512, cus);
    G = std::min<uint32_t>(std::max<uint32_t>(G, 1u), kMaxResidentWGs);
    if (cus > 0 && resident_fits(p.units, G, bf16)) return dispatch_resident<MODE>(p, bf16, vec, st, G, stream);
  }
  return dispatch_two_pass<MODE>(p, bf16, vec, batch, stream);
}

}  // namespace

hipError_t launch_quantize(QuantParams p, bool bf16, bool vec, uint32_t batch, ResidentState *st,
                           hipStream_t stream) {
  if (p.fp8) return dispatch<kFp8>(p, bf16, vec, batch, st, stream);
  if (p.four6) return dispatch<kFour6>(p, bf16, vec, batch, st, stream);  // offline weights: two-pass
  if (p.y) return dispatch<kQdq>(p, bf16, vec, batch, st, stream);
  return dispatch<kNvfp4>(p, bf16, vec, batch, st, stream);
}

}  // namespace nvfp4
