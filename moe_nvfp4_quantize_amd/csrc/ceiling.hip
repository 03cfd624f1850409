// ceiling.hip -- HBM ceiling kernels for the benchmark (libnvfp4_ceiling.so).
//
// Not part of the quantized layer: two streaming kernels that measure what
// this GPU's memory system delivers to a kernel with the quantizer's access
// pattern, so the quantizer's rate can be stated against a measured ceiling
// as well as against the 8 TB/s specification.
//
//  * read:        every 16-element unit (32 bytes of bf16) read once with
//                 non-temporal 16-byte loads, one XOR-sum per workgroup
//                 written out (so the loads are not removed);
//  * read_write:  the same reads, and per unit the quantizer's writes: 8 bytes
//                 to one array (codes) and 1 byte to another (scales), with
//                 non-temporal stores at the same addresses the quantizer
//                 writes.  Written values are the low bits of the data read.
// Both walk the units grid-stride, consecutive threads on consecutive units,
// UPT units per thread in flight; the host picks one workgroup per compute
// unit or more.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 512;

template <int UPT>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *__restrict__ x, uint64_t units,
                                                        uint32_t *__restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + (UPT - 1) * stride < units; u += UPT * stride) {
    u32x4 v[UPT][2];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      v[i][0] = __builtin_nontemporal_load(x + 2 * (u + i * stride));
      v[i][1] = __builtin_nontemporal_load(x + 2 * (u + i * stride) + 1);
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) acc ^= v[i][0][0] ^ v[i][0][3] ^ v[i][1][1] ^ v[i][1][2];
  }
  for (; u < units; u += stride) {
    const u32x4 a = __builtin_nontemporal_load(x + 2 * u), b = __builtin_nontemporal_load(x + 2 * u + 1);
    acc ^= a[0] ^ a[3] ^ b[1] ^ b[2];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t red[kThreads / 64];
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

template <int UPT>
__global__ __launch_bounds__(kThreads) void read_write_kernel(const u32x4 *__restrict__ x, uint64_t units,
                                                              uint64_t *__restrict__ q, uint8_t *__restrict__ s) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + (UPT - 1) * stride < units; u += UPT * stride) {
    u32x4 v[UPT][2];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      v[i][0] = __builtin_nontemporal_load(x + 2 * (u + i * stride));
      v[i][1] = __builtin_nontemporal_load(x + 2 * (u + i * stride) + 1);
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const uint64_t w = ((uint64_t)(v[i][0][0] ^ v[i][0][2] ^ v[i][1][0]) << 32) | (v[i][0][1] ^ v[i][1][3]);
      __builtin_nontemporal_store(w, q + u + i * stride);
      __builtin_nontemporal_store((uint8_t)(v[i][1][1] ^ v[i][0][3]), s + u + i * stride);
    }
  }
  for (; u < units; u += stride) {
    const u32x4 a = __builtin_nontemporal_load(x + 2 * u), b = __builtin_nontemporal_load(x + 2 * u + 1);
    __builtin_nontemporal_store(((uint64_t)(a[0] ^ a[2] ^ b[0]) << 32) | (a[1] ^ b[3]), q + u);
    __builtin_nontemporal_store((uint8_t)(b[1] ^ a[3]), s + u);
  }
}

uint32_t cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n > 0 ? (uint32_t)n : 0u;
}

}  // namespace

extern "C" {

// Workgroups the kernels below launch: wgs_per_cu per compute unit.
uint32_t ceiling_grid(uint32_t wgs_per_cu) { return cu_count() * wgs_per_cu; }

// Reads `bytes` (a multiple of 32, 16-byte aligned) from x; writes grid words
// to sink (ceiling_grid(wgs_per_cu) uint32).  Returns a hipError_t.
int ceiling_read(const void *x, uint64_t bytes, uint32_t *sink, uint32_t wgs_per_cu, hipStream_t stream) {
  const uint32_t grid = ceiling_grid(wgs_per_cu);
  if (!x || !sink || bytes % 32 || grid == 0) return (int)hipErrorInvalidValue;
  read_kernel<4><<<grid, kThreads, 0, stream>>>(static_cast<const u32x4 *>(x), bytes / 32, sink);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 32) from x and writes bytes/4 to q and bytes/32
// to s: the traffic of quantizing bf16 to NVFP4.  Returns a hipError_t.
int ceiling_read_write(const void *x, uint64_t bytes, void *q, void *s, uint32_t wgs_per_cu,
                       hipStream_t stream) {
  const uint32_t grid = ceiling_grid(wgs_per_cu);
  if (!x || !q || !s || bytes % 32 || grid == 0) return (int)hipErrorInvalidValue;
  read_write_kernel<4><<<grid, kThreads, 0, stream>>>(static_cast<const u32x4 *>(x), bytes / 32,
                                                      static_cast<uint64_t *>(q), static_cast<uint8_t *>(s));
  return (int)hipGetLastError();
}

}  // extern "C"
