// Dispatch bookkeeping entry points of the forward (internal to the library;
// not part of the C ABI).
#pragma once

#include "common.h"

namespace moe {

// Batches of at most this many (token, slot) pairs are permuted by one block.
constexpr int64_t kSmallPermutePairs = 4096;

// launch_permute that also writes the grouped GEMMs' tile lists from the
// offsets it computes, as launch_build_tiles would: groups of 1..small_max
// rows get one small tile each, larger ones big_m-row tiles; the tile counts
// go to num_small / num_big.  With split_small (P <= kSmallPermutePairs
// only), groups of small_max+1 .. 2*small_max rows get two small tiles
// instead (the caller knows that no group is larger).
hipError_t launch_permute_with_tiles(int64_t P, int32_t E, const int32_t* ids, int32_t* counts,
                                     int32_t* offsets, int32_t* row_to_pair,
                                     int32_t* pair_to_row, int32_t* chunk_scratch,
                                     int32_t small_max, int32_t big_m, bool split_small,
                                     Tile* small_tiles, int32_t* num_small, Tile* big_tiles,
                                     int32_t* num_big, hipStream_t s);

}  // namespace moe
