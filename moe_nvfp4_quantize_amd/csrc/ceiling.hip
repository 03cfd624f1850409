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
//
// And the matrix-core ceiling of the GEMM's arithmetic, with no memory or LDS
// traffic: one workgroup of four waves per compute unit, each wave a 128 x 128
// block of 4 x 4 accumulators of v_mfma_f32_32x32x16_f16 on operands held in
// registers (the GEMM's wave tile), either MFMAs alone or with the GEMM's exact
// FP4 -> f16 decode of the next sub-step's operands (4 converts and 4 packed
// multiplies per 8 codes, 8 fragments per 16 MFMAs) interleaved between them.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

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

// 8 codes of a dword times a block scale (s / 256, as the GEMM keeps it) -> 8 f16
__device__ __forceinline__ half8v decode8(uint32_t w, _Float16 s) {
  const half2v s2 = {s, s};
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s2;
  return (half8v){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// iters x 2 sub-steps of 16 MFMAs per wave; DECODE: the operands of the next
// sub-step decoded from codes that change every iteration (a scalar salt) while
// the current sub-step's MFMAs run, one MFMA then a few VALU instructions in turn
template <bool DECODE>
__global__ __launch_bounds__(256, 1) void mfma_kernel(float *__restrict__ sink, uint32_t iters) {
  constexpr int F = 4, NM = F * F, VPM = (9 * 2 * F + NM - 1) / NM;
  float16v acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const _Float16 sc = (_Float16)0.00390625f;
  uint32_t ca[F], cb[F];
  half8v av[2][F], bv[2][F];
#pragma unroll
  for (int i = 0; i < F; ++i) {
    ca[i] = (threadIdx.x * 2654435761u) ^ (0x9e3779b9u * (i + 1));
    cb[i] = (threadIdx.x * 2246822519u) ^ (0x85ebca6bu * (i + 1));
    av[0][i] = av[1][i] = decode8(ca[i], sc);
    bv[0][i] = bv[1][i] = decode8(cb[i], sc);
  }
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t salt = __builtin_amdgcn_readfirstlane(it * 0x01010101u);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[t][j], av[t][i], acc[i][j], 0, 0, 0);
      if constexpr (DECODE) {
#pragma unroll
        for (int i = 0; i < F; ++i) {
          av[t ^ 1][i] = decode8(ca[i] ^ salt ^ t, sc);
          bv[t ^ 1][i] = decode8(cb[i] ^ salt ^ t, sc);
        }
#pragma unroll
        for (int k = 0; k < NM; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

uint32_t ceiling_grid(uint32_t wgs_per_cu);

// Matrix-core ceiling: ceiling_grid(1) workgroups of 256 threads, each wave
// 2 x iters x 16 MFMAs of 32 x 32 x 16 (f16 in, f32 accumulate), with or
// without the exact FP4 decode in between; sink receives ceiling_grid(1) x 256
// floats.  Returns a hipError_t.
int ceiling_mfma(float *sink, uint32_t iters, int decode, hipStream_t stream) {
  const uint32_t grid = ceiling_grid(1);
  if (!sink || grid == 0 || iters == 0) return (int)hipErrorInvalidValue;
  if (decode)
    mfma_kernel<true><<<grid, 256, 0, stream>>>(sink, iters);
  else
    mfma_kernel<false><<<grid, 256, 0, stream>>>(sink, iters);
  return (int)hipGetLastError();
}

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
