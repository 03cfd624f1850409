// nvfp4_common.hpp -- small shared pieces of the gfx950 kernels and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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

// Compute units of the current device, cached per device (host; 0 when the
// query fails).  The cache is written with relaxed atomics: concurrent first
// calls store the same value.
inline uint32_t device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
    cache[dev].store(n, std::memory_order_relaxed);
    v = n;
  }
  return v > 0 ? (uint32_t)v : 0u;
}

// ------------------------------------------------------------ GEMM helpers

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Swizzle of the four 16-byte pieces of a 64-byte LDS row: piece c of row r
// is stored at c ^ swz(r).  A 16-byte read of 64 lanes is served 16 lanes
// (256 bytes, all 64 banks) at a time; in the fragment reads lane l reads
// piece c of row r0 + l % 32, so 16 consecutive rows must cover the 16
// distinct 16-byte slots of a 256-byte window: rows r % 4 give the 64-byte
// quarter, swz(r) = (r / 4) % 4 the piece inside it (measured on gfx950:
// no bank conflicts, where an unswizzled layout shows 3 of 4 LDS cycles lost).
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r >> 2) & 3u; }

// Which output tile dense workgroup w computes.  Workgroup w runs on XCD
// w % 8, so each XCD is given a contiguous range of tiles, swept 8 tile-rows
// at a time so that concurrently running workgroups share A and B tiles in
// that XCD's L2.
__device__ __forceinline__ void dense_tile(uint32_t w, uint32_t tiles_m, uint32_t tiles_n,
                                           uint32_t *tm, uint32_t *tn) {
  const uint32_t G = tiles_m * tiles_n;
  const uint32_t q = G / 8, r = G % 8, x = w % 8, local = w / 8;
  const uint32_t idx = x * q + min(x, r) + local;
  constexpr uint32_t GM = 8;
  const uint32_t group = idx / (GM * tiles_n);
  const uint32_t first_m = group * GM;
  const uint32_t gsize = min(tiles_m - first_m, GM);
  const uint32_t pid = idx - group * GM * tiles_n;
  *tm = first_m + pid % gsize;
  *tn = pid / gsize;
}

}  // namespace nvfp4
