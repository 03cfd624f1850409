// moe.hip -- routed-expert plumbing on gfx950: router top-k + softmax, the
// deterministic permutation of routed rows by expert, and the weighted combine.
//
// Qwen3.8-Flash-Next-NVFP4 page, section "Why only routed experts": each token
// is sent to k of E experts (top-10 of 512 there) picked by a BF16 router; only
// the routed experts' weights are NVFP4.
//
// Routing order: per token, experts by descending logit, equal logits by lower
// expert id.  Routed rows are grouped by expert and, inside an expert, by
// ascending token (a token never picks an expert twice).  The permutation is a
// counting sort with no order-dependent atomics, so it is identical run to run:
//   1. topk:   one wave per token; k rounds of a wave arg-max; softmax of the
//              k selected logits.
//   2. count:  one wave per group of 64 tokens; LDS bit masks mask[e] (bit L =
//              token L of the group picked e), counts[g][e] = popcount.
//   3. scan:   one workgroup; exclusive prefix of counts in (expert, group)
//              order -> base[g][e] and expert_offsets.
//   4. place:  one wave per group; the row of (token L, slot j) with expert e is
//              base[g][e] + popcount(mask[e] & bits below L).
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"

namespace nvfp4 {

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kPerLane = kMaxE / 64;

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, uint32_t T,
                                                   uint32_t E, uint32_t k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
  const uint32_t lane = threadIdx.x % 64;
  const uint32_t t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  const float *row = logits + (int64_t)t * E;
  float v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const uint32_t e = lane + 64u * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;  // bit i: expert lane + 64 i already selected
  float sel_v = 0.0f;  // lane j < k keeps the j-th selection
  int32_t sel_e = 0;
  for (uint32_t j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int32_t be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const uint32_t e = lane + 64u * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && (int32_t)e < be))) {
        bv = v[i];
        be = (int32_t)e;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int32_t oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((uint32_t)be % 64u == lane) taken |= 1u << ((uint32_t)be / 64u);
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
  }
  // softmax over the k selected logits; the first is the largest
  const float top = __shfl(sel_v, 0, 64);
  const float ex = lane < k ? expf(sel_v - top) : 0.0f;
  float sum = ex;
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = sel_e;
    w[(int64_t)t * k + lane] = ex / sum;
  }
}

// masks for the 64 tokens of group g, in LDS; returns nothing, fills mask[E]
__device__ void build_masks(unsigned long long *mask, const int32_t *ids, uint32_t T, uint32_t E,
                            uint32_t k, uint32_t g) {
  const uint32_t lane = threadIdx.x;
  for (uint32_t e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  const uint32_t t = g * 64 + lane;
  if (t < T)
    for (uint32_t j = 0; j < k; ++j) atomicOr(&mask[ids[(int64_t)t * k + j]], 1ull << lane);
  __syncthreads();
}

__global__ __launch_bounds__(64) void count_kernel(const int32_t *ids, uint32_t T, uint32_t E,
                                                   uint32_t k, int32_t *counts) {
  __shared__ unsigned long long mask[kMaxE];
  const uint32_t g = blockIdx.x;
  build_masks(mask, ids, T, E, k, g);
  for (uint32_t e = threadIdx.x; e < E; e += 64) counts[(int64_t)g * E + e] = __popcll(mask[e]);
}

// one workgroup of 1024 threads; counts[g][e] -> base[g][e] (in place) with the
// exclusive prefix taken in (e, g) order; offsets[e] = base[0][e], offsets[E] = R
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *counts, uint32_t G, uint32_t E,
                                                    int32_t *offsets) {
  __shared__ int32_t part[1024];
  const uint32_t n = G * E;
  const uint32_t per = (n + 1023) / 1024;
  const uint32_t lo = threadIdx.x * per, hi = min(lo + per, n);
  // element i of the (e, g) order is counts[g][e] with e = i / G, g = i % G
  int32_t s = 0;
  for (uint32_t i = lo; i < hi; ++i) s += counts[(int64_t)(i % G) * E + i / G];
  part[threadIdx.x] = s;
  __syncthreads();
  for (uint32_t off = 1; off < 1024; off <<= 1) {
    int32_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - s;
  for (uint32_t i = lo; i < hi; ++i) {
    int32_t *c = counts + (int64_t)(i % G) * E + i / G;
    const int32_t cnt = *c;
    *c = run;
    if (i % G == 0) offsets[i / G] = run;
    run += cnt;
  }
  if (threadIdx.x == 1023) offsets[E] = part[1023];
}

__global__ __launch_bounds__(64) void place_kernel(const int32_t *ids, uint32_t T, uint32_t E,
                                                   uint32_t k, const int32_t *base,
                                                   int32_t *src_row, int32_t *inv) {
  __shared__ unsigned long long mask[kMaxE];
  const uint32_t g = blockIdx.x;
  build_masks(mask, ids, T, E, k, g);
  const uint32_t lane = threadIdx.x;
  const uint32_t t = g * 64 + lane;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (uint32_t j = 0; j < k; ++j) {
    const int32_t e = ids[(int64_t)t * k + j];
    const int32_t r = base[(int64_t)g * E + e] + __popcll(mask[e] & below);
    src_row[r] = (int32_t)t;
    inv[(int64_t)t * k + j] = r;
  }
}

// out[t][h] = sum_j w[t][j] * y[inv[t][j]][h]; one workgroup per token, 4
// consecutive h per thread.
template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT *__restrict__ y,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv, uint32_t k,
                                                      uint32_t H, OT *__restrict__ out) {
  const uint32_t t = blockIdx.x;
  __shared__ int32_t rows[kMaxK];
  __shared__ float ws[kMaxK];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = inv[(int64_t)t * k + threadIdx.x];
    ws[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (uint32_t h = threadIdx.x; h < H; h += 256) {
    float acc = 0.0f;
    for (uint32_t j = 0; j < k; ++j) {
      float v;
      if constexpr (sizeof(YT) == 4)
        v = y[(int64_t)rows[j] * H + h];
      else
        v = u2f((uint32_t)y[(int64_t)rows[j] * H + h] << 16);
      acc += ws[j] * v;
    }
    if constexpr (sizeof(OT) == 4)
      out[(int64_t)t * H + h] = acc;
    else
      out[(int64_t)t * H + h] = (OT)float_to_bf16_bits(acc);
  }
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int32_t E, int32_t /*k*/) {
  const int64_t G = (T + 63) / 64;
  return (size_t)(G * E * 4 + 256);
}

hipError_t launch_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *topk_ids,
                        float *topk_w, int32_t *offsets, int32_t *src_row, int32_t *inv,
                        void *workspace, hipStream_t stream) {
  const uint32_t G = (uint32_t)((T + 63) / 64);
  int32_t *counts = static_cast<int32_t *>(workspace);
  if (T > 0) {
    topk_kernel<<<(uint32_t)((T + 3) / 4), 256, 0, stream>>>(logits, (uint32_t)T, (uint32_t)E,
                                                              (uint32_t)k, topk_ids, topk_w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    count_kernel<<<G, 64, 0, stream>>>(topk_ids, (uint32_t)T, (uint32_t)E, (uint32_t)k, counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  scan_kernel<<<1, 1024, 0, stream>>>(counts, G, (uint32_t)E, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  place_kernel<<<G, 64, 0, stream>>>(topk_ids, (uint32_t)T, (uint32_t)E, (uint32_t)k, counts,
                                     src_row, inv);
  return hipGetLastError();
}

hipError_t launch_combine(const void *y, bool y_bf16, const float *w, const int32_t *inv, int64_t T,
                          int32_t k, int64_t H, void *out, bool out_bf16, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((uint32_t)T);
  if (y_bf16) {
    if (out_bf16)
      combine_kernel<uint16_t, uint16_t><<<grid, 256, 0, stream>>>(
          (const uint16_t *)y, w, inv, k, (uint32_t)H, (uint16_t *)out);
    else
      combine_kernel<uint16_t, float><<<grid, 256, 0, stream>>>((const uint16_t *)y, w, inv, k,
                                                                (uint32_t)H, (float *)out);
  } else {
    if (out_bf16)
      combine_kernel<float, uint16_t><<<grid, 256, 0, stream>>>((const float *)y, w, inv, k,
                                                                (uint32_t)H, (uint16_t *)out);
    else
      combine_kernel<float, float><<<grid, 256, 0, stream>>>((const float *)y, w, inv, k,
                                                             (uint32_t)H, (float *)out);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
