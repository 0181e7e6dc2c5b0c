// Router logits of small batches with K split over workgroups (internal to
// the library; not part of the C ABI).
#pragma once

#include "common.h"

namespace moe {

// Batches of at most this many tokens take the split product.
constexpr int64_t kRouterSplitMaxT = 256;

// K slices of the split product for E experts and hidden width H: whole
// 32-deep steps, at most 8 per slice.
int router_splits(int E, int H);

// part[s][t][e] = sum over k in slice s of x[t, k] * w[e, k] (bf16 inputs,
// fp32 sums), then logits[t][e] = sum_s part[s][t][e] (+ bias[e]) in slice
// order.  T <= kRouterSplitMaxT, E <= kMaxExperts, H a multiple of 32;
// part holds router_splits(E, H) * T * E floats.
hipError_t launch_router_split(const bf16_t* x, int64_t T, int H, const bf16_t* w, int E,
                               const float* bias, float* part, float* logits, hipStream_t s);

}  // namespace moe
