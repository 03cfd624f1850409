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
//   3. scan:   one workgroup; per expert, the exclusive prefix of its counts
//              over the groups -> base[g][e] (in place), and the exclusive
//              prefix of the experts' totals -> expert_offsets.
//   4. place:  one wave per group; the row of (token L, slot j) with expert e is
//              expert_offsets[e] + base[g][e] + popcount(mask[e] & bits below L).
#include "nvfp4_common.hpp"
#include "nvfp4_format.hpp"
#include "nvfp4_kernels.hpp"
#include "moe_select.hpp"

namespace nvfp4 {

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxPerLane = kMaxE / 64;

// PL = logits per lane (E <= 64 PL)
template <int PL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, uint32_t T,
                                                   uint32_t E, uint32_t k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
  const uint32_t lane = threadIdx.x % 64;
  const uint32_t t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  const float *row = logits + (int64_t)t * E;
  float v[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const uint32_t e = lane + 64u * i;
    v[i] = e < E ? router_logit(row[e]) : -INFINITY;
  }
  // bit i: expert lane + 64 i is selectable (exists, not yet selected)
  uint32_t open = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) open |= (lane + 64u * i < E ? 1u : 0u) << i;
  float sel_v = 0.0f;  // lane j < k keeps the j-th selection
  int32_t sel_e = 0;
  for (uint32_t j = 0; j < k; ++j) {
    // candidates compared without branches: larger value first, then lower id
    float bv = -INFINITY;
    int32_t be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int32_t e = (int32_t)(lane + 64u * i);
      const bool take = ((open >> i) & 1u) & topk_before(v[i], e, bv, be);
      bv = take ? v[i] : bv;
      be = take ? e : be;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int32_t oe = __shfl_xor(be, off, 64);
      const bool take = topk_before(ov, oe, bv, be);
      bv = take ? ov : bv;
      be = take ? oe : be;
    }
    if ((uint32_t)be % 64u == lane) open &= ~(1u << ((uint32_t)be / 64u));
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

// One workgroup of 1024 threads.  Thread e < E walks expert e's column of
// counts[g][e] (coalesced across the threads) and replaces it in place by its
// exclusive prefix over g; the column totals are then scanned over e into
// offsets (offsets[e] = first row of expert e, offsets[E] = R).  The routed row
// of group g's first token with expert e is offsets[e] + counts[g][e].
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *counts, uint32_t G, uint32_t E,
                                                    int32_t *offsets) {
  __shared__ int32_t part[16];
  const uint32_t e = threadIdx.x, lane = e % 64, wv = e / 64;
  int32_t run = 0;
  if (e < E) {
    uint32_t g = 0;
    // 32 loads in flight per thread: the column walk is a chain of memory latencies
    for (; g + 32 <= G; g += 32) {
      int32_t c[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = counts[(int64_t)(g + i) * E + e];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        counts[(int64_t)(g + i) * E + e] = run;
        run += c[i];
      }
    }
    for (; g + 8 <= G; g += 8) {
      int32_t c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = counts[(int64_t)(g + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        counts[(int64_t)(g + i) * E + e] = run;
        run += c[i];
      }
    }
    for (; g < G; ++g) {
      const int32_t c = counts[(int64_t)g * E + e];
      counts[(int64_t)g * E + e] = run;
      run += c;
    }
  }
  // exclusive scan of the column totals over e: inside each wave, then the
  // sixteen wave totals through LDS (threads e >= E contribute 0)
  int32_t incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(incl, off, 64);
    if (lane >= (uint32_t)off) incl += v;
  }
  if (lane == 63) part[wv] = incl;
  __syncthreads();
  int32_t before = 0;
  for (uint32_t w = 0; w < wv; ++w) before += part[w];
  if (e < E) offsets[e] = before + incl - run;
  if (e == 1023) offsets[E] = before + incl;
}

__global__ __launch_bounds__(64) void place_kernel(const int32_t *ids, uint32_t T, uint32_t E,
                                                   uint32_t k, const int32_t *base,
                                                   const int32_t *offsets, int32_t *src_row,
                                                   int32_t *inv) {
  __shared__ unsigned long long mask[kMaxE];
  const uint32_t g = blockIdx.x;
  build_masks(mask, ids, T, E, k, g);
  const uint32_t lane = threadIdx.x;
  const uint32_t t = g * 64 + lane;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (uint32_t j = 0; j < k; ++j) {
    const int32_t e = ids[(int64_t)t * k + j];
    const int32_t r = offsets[e] + base[(int64_t)g * E + e] + __popcll(mask[e] & below);
    src_row[r] = (int32_t)t;
    inv[(int64_t)t * k + j] = r;
  }
}

// out[t][h] = sum_j w[t][j] * y[inv[t][j]][h], slots in order, one product and
// one float32 addition per slot (no fused multiply-add); one workgroup per token.
// VEC (H % 8 == 0, 16-byte aligned y and out): each thread owns 8 consecutive h
// and loads them 16 (bf16) or 32 (f32) bytes at a time, four slots' loads in
// flight before they are summed; otherwise one h per thread.
template <typename YT>
__device__ __forceinline__ void load8(const YT *p, float v[8]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (sizeof(YT) == 4) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(p), b = *reinterpret_cast<const u32x4 *>(p + 4);
    for (int i = 0; i < 4; ++i) {
      v[i] = u2f(a[i]);
      v[4 + i] = u2f(b[i]);
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(a[i]);
      v[2 * i + 1] = bf16_hi(a[i]);
    }
  }
}

template <typename OT>
__device__ __forceinline__ void store8(OT *p, const float v[8]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (sizeof(OT) == 4) {
    *reinterpret_cast<u32x4 *>(p) = (u32x4){f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])};
    *reinterpret_cast<u32x4 *>(p + 4) = (u32x4){f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7])};
  } else {
    u32x4 o;
    for (int i = 0; i < 4; ++i) o[i] = float_to_bf16_bits(v[2 * i]) | (float_to_bf16_bits(v[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4 *>(p) = o;
  }
}

template <typename YT, typename OT, bool VEC>
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
  if constexpr (VEC) {
    for (uint32_t h = threadIdx.x * 8; h < H; h += 256 * 8) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      uint32_t j = 0;
      for (; j + 4 <= k; j += 4) {
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) load8<YT>(y + (int64_t)rows[j + q] * H + h, v[q]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += ws[j + q] * v[q][i];
      }
      for (; j < k; ++j) {
        float v[8];
        load8<YT>(y + (int64_t)rows[j] * H + h, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += ws[j] * v[i];
      }
      store8<OT>(out + (int64_t)t * H + h, acc);
    }
  } else {
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
}

template <typename YT, typename OT>
hipError_t launch_combine_t(const void *y, const float *w, const int32_t *inv, int64_t T, int32_t k,
                            int64_t H, void *out, hipStream_t stream) {
  const bool vec = H % 8 == 0 && ((uintptr_t)y & 15u) == 0 && ((uintptr_t)out & 15u) == 0;
  if (vec)
    combine_kernel<YT, OT, true><<<(uint32_t)T, 256, 0, stream>>>((const YT *)y, w, inv, (uint32_t)k,
                                                                  (uint32_t)H, (OT *)out);
  else
    combine_kernel<YT, OT, false><<<(uint32_t)T, 256, 0, stream>>>((const YT *)y, w, inv, (uint32_t)k,
                                                                   (uint32_t)H, (OT *)out);
  return hipGetLastError();
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
    const uint32_t grid = (uint32_t)((T + 3) / 4);
    if (E <= 128)
      topk_kernel<2><<<grid, 256, 0, stream>>>(logits, (uint32_t)T, (uint32_t)E, (uint32_t)k, topk_ids, topk_w);
    else if (E <= 256)
      topk_kernel<4><<<grid, 256, 0, stream>>>(logits, (uint32_t)T, (uint32_t)E, (uint32_t)k, topk_ids, topk_w);
    else if (E <= 512)
      topk_kernel<8><<<grid, 256, 0, stream>>>(logits, (uint32_t)T, (uint32_t)E, (uint32_t)k, topk_ids, topk_w);
    else
      topk_kernel<kMaxPerLane><<<grid, 256, 0, stream>>>(logits, (uint32_t)T, (uint32_t)E, (uint32_t)k, topk_ids,
                                                      topk_w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    count_kernel<<<G, 64, 0, stream>>>(topk_ids, (uint32_t)T, (uint32_t)E, (uint32_t)k, counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  scan_kernel<<<1, 1024, 0, stream>>>(counts, G, (uint32_t)E, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  place_kernel<<<G, 64, 0, stream>>>(topk_ids, (uint32_t)T, (uint32_t)E, (uint32_t)k, counts,
                                     offsets, src_row, inv);
  return hipGetLastError();
}

hipError_t launch_combine(const void *y, bool y_bf16, const float *w, const int32_t *inv, int64_t T,
                          int32_t k, int64_t H, void *out, bool out_bf16, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (y_bf16)
    return out_bf16 ? launch_combine_t<uint16_t, uint16_t>(y, w, inv, T, k, H, out, stream)
                    : launch_combine_t<uint16_t, float>(y, w, inv, T, k, H, out, stream);
  return out_bf16 ? launch_combine_t<float, uint16_t>(y, w, inv, T, k, H, out, stream)
                  : launch_combine_t<float, float>(y, w, inv, T, k, H, out, stream);
}

}  // namespace nvfp4
