// nvfp4_common.hpp -- small shared pieces of the gfx950 kernels and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Unsigned 32-bit division by a run-time constant d >= 1 through a multiply and
// a shift (round-up reciprocal method): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (umulhi(n, m) + n) >> l for every
// 32-bit n (the sum is formed in 64 bits).
struct FastDiv {
  uint32_t d, m, l;
  FastDiv() : d(1), m(0), l(0) {}
  explicit FastDiv(uint32_t divisor) : d(divisor) {
    l = 0;
    while ((1ull << l) < divisor) ++l;
    m = (uint32_t)(((1ull << 32) * ((1ull << l) - divisor)) / divisor + 1);
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    uint64_t hi = ((uint64_t)n * m) >> 32;
    return (uint32_t)((hi + n) >> l);
  }
};

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Block-wide max over blockDim.x threads (a multiple of 64, at most 1024);
// every thread gets the result.
__device__ __forceinline__ float block_max(float v) {
  __shared__ float red[16];
  v = wave_max(v);
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // red[] may still be read by a previous call
  if (lane == 0) red[wid] = v;
  __syncthreads();
  const int nw = blockDim.x >> 6;
  float r = lane < nw ? red[lane] : 0.0f;
  return wave_max(r);
}

}  // namespace nvfp4
