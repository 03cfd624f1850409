// moe_select.hpp -- the router's top-k comparison, shared by the top-k kernel
// and its host check.
//
// Qwen3.8-Flash-Next-NVFP4 page, section "Why only routed experts": each token
// goes to the k experts with the largest router logits.  Order: larger logit
// first, equal logits by lower expert id.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// The logit a candidate is ranked by.  A NaN compares false against
// everything, so it would never be selected and a row with fewer than k
// non-NaN logits would run out of candidates; it is ranked as -infinity
// instead (below every finite logit, tied with -infinity, ties by lower id),
// so every round selects an existing, not yet selected expert.
__host__ __device__ __forceinline__ float router_logit(float x) {
  return x != x ? -__builtin_inff() : x;
}

// Whether candidate (v, e) ranks before (bv, be).  The initial best of a round
// is (-infinity, INT32_MAX): any existing candidate, -infinity included, ranks
// before it through the lower id.
__host__ __device__ __forceinline__ bool topk_before(float v, int32_t e, float bv, int32_t be) {
  return (v > bv) | ((v == bv) & (e < be));
}

}  // namespace nvfp4
