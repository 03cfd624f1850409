// quantize.hip -- dynamic / static two-level NVFP4 quantization on gfx950.
//
// Qwen3.8-Flash-Next-NVFP4 page, section "Core: the W4A4 two-level scaling
// mechanism" (level 1: one E4M3 scale per 16 elements along the last dimension;
// level 2: one FP32 scale per tensor) and sub-section "The A4 side: dynamic
// activations" (activations quantized on the fly with the same rule).
//
// Two passes over the input:
//   1. amax_partials: each workgroup reduces max|x| over a strided share of the
//      16-element blocks and writes one partial per workgroup (no atomics, so no
//      zero-initialised state is needed and the result is order independent);
//   2. quantize: each workgroup first reduces the partials to amax and forms
//      g = amax / 2688 (workgroup 0 stores it), then every thread encodes whole
//      16-element blocks: block max, E4M3 block scale, one reciprocal, 16 E2M1
//      codes packed into 8 bytes.
// A thread owns a whole block, so the block max needs no cross-lane traffic;
// consecutive threads own consecutive blocks of a row, so each wave reads
// 2 KB (bf16) or 4 KB (fp32) of contiguous input and writes 512 B of codes and
// 64 B of scales.
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

// 16 consecutive elements starting at p.  VEC: p is 16-byte aligned.
template <typename T, bool VEC>
__device__ __forceinline__ void load_block(const T *p, float v[16]);

template <>
__device__ __forceinline__ void load_block<uint16_t, true>(const uint16_t *p, float v[16]) {
  const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
  const uint4 a = p4[0];
  const uint4 b = p4[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void load_block<uint16_t, false>(const uint16_t *p, float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = u2f((uint32_t)p[i] << 16);
}

template <>
__device__ __forceinline__ void load_block<float, true>(const float *p, float v[16]) {
  const float4 *p4 = reinterpret_cast<const float4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 t = p4[i];
    v[4 * i] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

template <>
__device__ __forceinline__ void load_block<float, false>(const float *p, float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = p[i];
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(QuantParams p) {
  const uint32_t b = blockIdx.y;
  const T *x = static_cast<const T *>(p.x) + (int64_t)b * p.x_mstride;
  float m = 0.0f;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < p.units; u += gridDim.x * kThreads) {
    const uint32_t row = p.div_nbpr.div(u);
    const uint32_t blk = u - row * p.nbpr;
    float v[16];
    load_block<T, VEC>(x + (int64_t)row * p.ld + blk * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = block_max(m);
  if (threadIdx.x == 0) p.partials[(int64_t)b * p.P + blockIdx.x] = m;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
  const uint32_t b = blockIdx.y;
  float g;
  if (p.static_global) {
    g = p.g[b];
  } else {
    float m = 0.0f;
    for (uint32_t i = threadIdx.x; i < p.P; i += kThreads) m = fmaxf(m, p.partials[(int64_t)b * p.P + i]);
    m = block_max(m);
    g = m > 0.0f ? m / kGlobalDivisor : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) p.g[b] = g;
  }
  const float six_g = 6.0f * g;

  const T *x = static_cast<const T *>(p.x) + (int64_t)b * p.x_mstride;
  uint8_t *q = p.q + (int64_t)b * p.q_mstride;
  uint8_t *s = p.s + (int64_t)b * p.s_mstride;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < p.units; u += gridDim.x * kThreads) {
    const uint32_t row = p.div_nbpr.div(u);
    const uint32_t blk = u - row * p.nbpr;
    float v[16];
    load_block<T, VEC>(x + (int64_t)row * p.ld + blk * 16, v);
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(v[i]));
    float r;
    const uint32_t sc = block_scale(bmax, six_g, g, &r);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo |= e2m1_encode(v[i] * r) << (4 * i);
      hi |= e2m1_encode(v[8 + i] * r) << (4 * i);
    }
    // u == row * nbpr + blk, and q/s rows are dense: offsets are u*8 and u
    *reinterpret_cast<uint2 *>(q + (int64_t)u * 8) = make_uint2(lo, hi);
    s[u] = (uint8_t)sc;
  }
}

template <typename T, bool VEC>
hipError_t launch_typed(const QuantParams &p, uint32_t batch, uint32_t qgrid, hipStream_t stream) {
  if (!p.static_global) {
    amax_partials_kernel<T, VEC><<<dim3(p.P, batch), kThreads, 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  quantize_kernel<T, VEC><<<dim3(qgrid, batch), kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

uint32_t quantize_partials_per_matrix(uint64_t units) {
  uint64_t wg = (units + kThreads - 1) / kThreads;
  if (wg < 1) wg = 1;
  return (uint32_t)(wg < kMaxPartials ? wg : kMaxPartials);
}

hipError_t launch_quantize(QuantParams p, bool bf16, bool vec, uint32_t batch, hipStream_t stream) {
  uint64_t wg = ((uint64_t)p.units + kThreads - 1) / kThreads;
  if (wg < 1) wg = 1;
  // enough workgroups to fill the chip several times; each reduces P partials
  const uint32_t qgrid = (uint32_t)(wg < 2048 ? wg : 2048);
  if (bf16)
    return vec ? launch_typed<uint16_t, true>(p, batch, qgrid, stream)
               : launch_typed<uint16_t, false>(p, batch, qgrid, stream);
  return vec ? launch_typed<float, true>(p, batch, qgrid, stream)
             : launch_typed<float, false>(p, batch, qgrid, stream);
}

}  // namespace nvfp4
