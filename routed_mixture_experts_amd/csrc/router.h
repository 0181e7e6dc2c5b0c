// Dense products whose natural grids would leave CUs idle, with K split over
// workgroups and the slices summed in order: the router logits (small
// batches in a dedicated kernel, larger ones in 128x128 tiles) and the
// latent down-projection (internal to the library; not part of the C ABI).
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

// Larger batches whose 128x128 tile grid would leave CUs idle: K split over
// the second grid dimension of the 128x128 kernel (1 when the grid is large
// enough).
int router_tiled_splits(int64_t T, int E, int H);

// The same product with router_tiled_splits(T, E, H) > 1 slices, the slices
// summed in order with the bias; part holds that many T x E floats.
hipError_t launch_router_tiled(const bf16_t* x, int64_t T, int H, const bf16_t* w, int E,
                               const float* bias, float* part, float* logits, hipStream_t s);

// Floats of partial sums either split product needs for any T <= max_T.
size_t router_part_floats(int64_t max_T, int E, int H);

// Dense bf16 products C[T, N] = A[T, K] . B[N, K]^T whose 128x128 grid would
// leave CUs idle (under 384 tiles): K split into dense_tiled_splits(T, N, K)
// slices (1: not split), the slices summed in order and rounded once to
// bf16.  part holds that many T x N floats; dense_part_floats bounds it for
// any T <= max_T.  N a multiple of 4.
int dense_tiled_splits(int64_t T, int N, int K);
hipError_t launch_dense_sliced_bf16(const bf16_t* A, int64_t T, int K, const bf16_t* B, int N,
                                    float* part, bf16_t* out, hipStream_t s);
size_t dense_part_floats(int64_t max_T, int N, int K);

// A dense fp32 product (g.epi == EPI_F32, no tile list) in 128x128 tiles
// with K split into kslices: slice s writes its partial sums to
// C + s * M * ldc.  Defined with the kernel in gemm.hip.
hipError_t launch_tiled_kslices(const GemmArgs& g, int kslices, hipStream_t s);

}  // namespace moe
