// Dispatch bookkeeping: per-expert counts, their exclusive prefix sum, and a
// stable expert-sorted order of the (token, slot) pairs.
//
// "vLLM-Ascend Kimi K3 MoE Forward Insight", Stage 4 (mode table, AllGather
// row): dispatch sorts tokens by expert and returns the expert token counts;
// Stage 6: that list is per-expert counts or cumulative -- both are produced.
//
// Three small kernels, deterministic by construction (LDS atomics only count;
// no atomic decides a position), or one block for small batches (perm_small):
//   count   -- one block per chunk of 4096 pairs builds the chunk's histogram;
//   scan    -- one block turns the chunk histograms into per-(chunk, expert)
//              base rows, and writes counts and offsets;
//   scatter -- one block of 16 waves per chunk: each wave owns a contiguous
//              segment of the chunk and counts it per expert, the block
//              turns the chunk's base rows into per-wave bases, and each wave
//              walks its segment in order, 64 pairs at a time; lanes holding
//              the same expert find each other with one ballot per id bit (a
//              wave-wide multi-split), take their rank among lower lanes, and
//              the lowest of them advances the expert's running row in LDS.
// A fourth kernel turns the offsets into the tile list of a grouped GEMM.
#include "permute.h"

namespace moe {

namespace {

constexpr int kChunk = 4096;

__global__ __launch_bounds__(256) void perm_count(const int32_t* __restrict__ ids, int64_t P,
                                                   int E, int32_t* __restrict__ chunk_counts) {
    __shared__ int hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
        int64_t p = base + i;
        if (p < P) atomicAdd(&hist[ids[p]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of one int per thread across a block of whole waves (every
// block here has 1024 threads): a shuffle scan inside each wave, then the
// wave totals through LDS.  Integer sums, so the result does not depend on
// the order.  sh holds at least one int per wave.
__device__ int block_exclusive_scan(int v, int* sh, int& total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < nwaves; ++w) {
        const int t = sh[w];
        if (w < wave) base += t;
        all += t;
    }
    total = all;
    __syncthreads();  // sh is free for the next scan
    return base + x - v;
}

// Tile lists of the grouped GEMMs (optional kernel output: small_tiles != null).
struct TileOut {
    int32_t small_max, big_m, split_small;
    Tile* small_tiles;
    int32_t* num_small;
    Tile* big_tiles;
    int32_t* num_big;
};

// The tile lists of build_tiles_kernel, written by a block that has just
// computed every expert's row count (run) and first row (off), one thread
// per expert (tid < E).  Groups of 1..small_max rows get one small tile,
// with split_small groups of small_max+1 .. 2*small_max rows two, and the
// rest big_m-row big tiles.  Every thread of the block calls it (it scans).
__device__ void write_tiles(int tid, int E, int run, int off, const TileOut& tiles, int* sh) {
    if (!tiles.small_tiles) return;  // uniform over the block
    const int sm = tiles.small_max;
    const int ns = run <= 0 ? 0
                   : run <= sm ? 1
                   : tiles.split_small && run <= 2 * sm ? 2 : 0;
    const int nb = ns > 0 || tid >= E ? 0 : (run + tiles.big_m - 1) / tiles.big_m;
    int total_s, total_b;
    const int start_s = block_exclusive_scan(ns, sh, total_s);
    const int start_b = block_exclusive_scan(nb, sh, total_b);
    for (int i = 0; i < ns; ++i) {
        Tile t = {};
        t.group = tid;
        t.row0 = off + i * sm;
        t.row1 = min(off + (i + 1) * sm, off + run);
        t.first = start_s;
        t.count = ns;
        tiles.small_tiles[start_s + i] = t;
    }
    for (int i = 0; i < nb; ++i) {
        Tile t = {};
        t.group = tid;
        t.row0 = off + i * tiles.big_m;
        t.row1 = min(off + (i + 1) * tiles.big_m, off + run);
        t.first = start_b;
        t.count = nb;
        tiles.big_tiles[start_b + i] = t;
    }
    if (tid == 0) {
        *tiles.num_small = total_s;
        *tiles.num_big = total_b;
    }
}

__global__ __launch_bounds__(1024) void perm_scan(int nchunk, int E, int32_t* __restrict__ cc,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets, TileOut tiles) {
    __shared__ int sh[1024];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        // four chunks' counts are loaded before they are summed
        for (int c0 = 0; c0 < nchunk; c0 += 4) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = c0 + u < nchunk ? cc[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (c0 + u < nchunk) cc[(int64_t)(c0 + u) * E + e] = run;
                run += v[u];
            }
        }
    }
    int total;
    int off = block_exclusive_scan(e < E ? run : 0, sh, total);
    if (e < E) {
        counts[e] = run;
        offsets[e] = off;
        for (int c = 0; c < nchunk; ++c) cc[(int64_t)c * E + e] += off;
    }
    if (e == 0) offsets[E] = total;
    write_tiles(e, E, e < E ? run : 0, off, tiles, sh);
}

constexpr int kScatterWaves = 16;

// Per-wave segments of a chunk: whole 64-pair steps.
__device__ __forceinline__ int segment_len(int n) {
    return ((n + kScatterWaves * 64 - 1) / (kScatterWaves * 64)) * 64;
}

// Wave `wave` scatters pairs [p0, p1) in order from its cursors cur[id]
// (advanced as it goes): row = cursor + rank among lower lanes with the same
// id, found by one ballot per id bit.
__device__ __forceinline__ void scatter_segment(const int32_t* __restrict__ ids, int64_t p0,
                                                int64_t p1, int nbits, int* cur,
                                                int32_t* __restrict__ row_to_pair,
                                                int32_t* __restrict__ pair_to_row) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t s = p0; s < p1; s += 64) {
        const int64_t p = s + lane;
        const bool valid = p < p1;
        const int id = valid ? ids[p] : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (id >> b) & 1;
            const uint64_t bb = __ballot(valid && bit);
            peers &= bit ? bb : ~bb;
        }
        const int rank = __popcll(peers & below);
        const int cnt = __popcll(peers);
        // every lane reads its expert's cursor before the lowest peer moves
        // it (one LDS read, then one LDS write, in order within the wave)
        const int b0 = valid ? cur[id] : 0;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            const int row = b0 + rank;
            row_to_pair[row] = (int32_t)p;
            pair_to_row[p] = row;
            if (rank == 0) cur[id] = b0 + cnt;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

__global__ __launch_bounds__(1024) void perm_scatter(const int32_t* __restrict__ ids, int64_t P,
                                                     int E, int nbits,
                                                     const int32_t* __restrict__ chunk_base,
                                                     int32_t* __restrict__ row_to_pair,
                                                     int32_t* __restrict__ pair_to_row) {
    __shared__ int cur[kScatterWaves][kMaxExperts];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kScatterWaves * E; i += 1024) cur[i / E][i % E] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
    const int n = (int)min((int64_t)kChunk, P - c0);
    const int seg = segment_len(n);
    const int64_t p0 = c0 + min(wave * seg, n), p1 = c0 + min((wave + 1) * seg, n);
    for (int64_t p = p0 + lane; p < p1; p += 64) atomicAdd(&cur[wave][ids[p]], 1);
    __syncthreads();
    if (tid < E) {
        int run = chunk_base[(int64_t)blockIdx.x * E + tid];
#pragma unroll
        for (int w = 0; w < kScatterWaves; ++w) {
            const int c = cur[w][tid];
            cur[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    scatter_segment(ids, p0, p1, nbits, cur[wave], row_to_pair, pair_to_row);
}

// The whole permute of a small batch (P <= kSmallPairs) in one block of 16
// waves.  Wave w owns the contiguous pair segment [w * seg, (w + 1) * seg):
// it counts its pairs per expert (LDS atomics only count); one thread per
// expert turns the 16 segment counts into running bases, the block scans
// the expert totals into offsets, and each wave then scatters its segment
// in order with the ballot multi-split of perm_scatter, from its own
// per-expert cursors.  Segments are ordered by pair index, so rows inside
// an expert stay in ascending pair order -- the same result as the three
// kernels above.
constexpr int64_t kSmallPairs = kChunk;
static_assert(kSmallPairs == kSmallPermutePairs, "single-block permute limit");


__global__ __launch_bounds__(1024) void perm_small(const int32_t* __restrict__ ids, int P, int E,
                                                   int nbits, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ row_to_pair,
                                                   int32_t* __restrict__ pair_to_row,
                                                   TileOut tiles) {
    __shared__ int cur[kScatterWaves][kMaxExperts];
    __shared__ int sh[1024];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kScatterWaves * E; i += 1024) cur[i / E][i % E] = 0;
    __syncthreads();
    const int seg = segment_len(P);
    const int p0 = min(wave * seg, P), p1 = min((wave + 1) * seg, P);
    for (int p = p0 + lane; p < p1; p += 64) atomicAdd(&cur[wave][ids[p]], 1);
    __syncthreads();
    int run = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < kScatterWaves; ++w) {
            const int c = cur[w][tid];
            cur[w][tid] = run;
            run += c;
        }
    }
    int total;
    const int off = block_exclusive_scan(tid < E ? run : 0, sh, total);
    if (tid < E) {
        counts[tid] = run;
        offsets[tid] = off;
#pragma unroll
        for (int w = 0; w < kScatterWaves; ++w) cur[w][tid] += off;
    }
    if (tid == 0) offsets[E] = total;
    write_tiles(tid, E, run, off, tiles, sh);
    __syncthreads();
    scatter_segment(ids, p0, p1, nbits, cur[wave], row_to_pair, pair_to_row);
}

// Groups with 1..small_max rows get one tile each in the small list; larger
// groups are cut into big_m-row tiles in the big list.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int small_max, int big_m,
                                                           Tile* __restrict__ small_tiles,
                                                           int32_t* __restrict__ num_small,
                                                           Tile* __restrict__ big_tiles,
                                                           int32_t* __restrict__ num_big) {
    __shared__ int sh[1024];
    const int e = threadIdx.x;
    const int a = e < E ? offsets[e] : 0;
    const int b = e < E ? offsets[e + 1] : 0;
    const int c = b - a;
    const bool small = c > 0 && c <= small_max;
    const int nb = small ? 0 : (c + big_m - 1) / big_m;
    int total_s, total_b;
    const int start_s = block_exclusive_scan(small ? 1 : 0, sh, total_s);
    const int start_b = block_exclusive_scan(nb, sh, total_b);
    if (small) {
        Tile t = {};
        t.group = e;
        t.row0 = a;
        t.row1 = b;
        t.first = start_s;
        t.count = 1;
        small_tiles[start_s] = t;
    }
    for (int i = 0; i < nb; ++i) {
        Tile t = {};
        t.group = e;
        t.row0 = a + i * big_m;
        t.row1 = min(a + (i + 1) * big_m, b);
        t.first = start_b;
        t.count = nb;
        big_tiles[start_b + i] = t;
    }
    if (e == 0) {
        *num_small = total_s;
        *num_big = total_b;
    }
}

// Logical -> physical expert slot of every (token, slot) pair ("vLLM-Ascend
// Kimi K3 MoE Forward Insight", Stage 4: dispatch maps the logical topk_ids
// through log2phy when dynamic placement is active).  Out-of-range ids or
// table entries are clamped, so a stale table cannot index outside the
// weights.
__global__ __launch_bounds__(256) void log2phy_kernel(int64_t P, const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ log2phy,
                                                      int32_t num_logical, int32_t num_physical,
                                                      int32_t* __restrict__ phys) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    const int l = min(max(ids[p], 0), num_logical - 1);
    phys[p] = min(max(log2phy[l], 0), num_physical - 1);
}

// load[e] += counts[e] (Stage 6: the dispatch's per-expert token counts are
// added into the layer's EPLB load).
__global__ __launch_bounds__(256) void load_accumulate_kernel(int32_t n,
                                                              const int32_t* __restrict__ counts,
                                                              int64_t* __restrict__ load) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n) load[e] += counts[e];
}

}  // namespace

hipError_t launch_log2phy(int64_t P, const int32_t* ids, const int32_t* log2phy,
                          int32_t num_logical, int32_t num_physical, int32_t* phys,
                          hipStream_t s) {
    if (P > 0)
        log2phy_kernel<<<(unsigned)((P + 255) / 256), 256, 0, s>>>(P, ids, log2phy, num_logical,
                                                                    num_physical, phys);
    return hipGetLastError();
}

hipError_t launch_load_accumulate(int32_t n, const int32_t* counts, int64_t* load, hipStream_t s) {
    if (n > 0) load_accumulate_kernel<<<(n + 255) / 256, 256, 0, s>>>(n, counts, load);
    return hipGetLastError();
}

int permute_chunks(int64_t P) { return (int)((P + kChunk - 1) / kChunk); }

namespace {

hipError_t permute_impl(int64_t P, int32_t E, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* row_to_pair, int32_t* pair_to_row,
                        int32_t* chunk_scratch, const TileOut& tiles, hipStream_t s) {
    const int nchunk = permute_chunks(P);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    if (P <= kSmallPairs) {
        perm_small<<<1, 1024, 0, s>>>(ids, (int)P, E, nbits, counts, offsets, row_to_pair,
                                      pair_to_row, tiles);
        return hipGetLastError();
    }
    if (nchunk > 0) perm_count<<<nchunk, 256, 0, s>>>(ids, P, E, chunk_scratch);
    perm_scan<<<1, 1024, 0, s>>>(nchunk, E, chunk_scratch, counts, offsets, tiles);
    if (nchunk > 0)
        perm_scatter<<<nchunk, 1024, 0, s>>>(ids, P, E, nbits, chunk_scratch, row_to_pair,
                                             pair_to_row);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_permute(int64_t P, int32_t E, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* row_to_pair, int32_t* pair_to_row,
                          int32_t* chunk_scratch, hipStream_t s) {
    return permute_impl(P, E, ids, counts, offsets, row_to_pair, pair_to_row, chunk_scratch,
                        TileOut{}, s);
}

hipError_t launch_permute_with_tiles(int64_t P, int32_t E, const int32_t* ids, int32_t* counts,
                                     int32_t* offsets, int32_t* row_to_pair,
                                     int32_t* pair_to_row, int32_t* chunk_scratch,
                                     int32_t small_max, int32_t big_m, bool split_small,
                                     Tile* small_tiles, int32_t* num_small, Tile* big_tiles,
                                     int32_t* num_big, hipStream_t s) {
    if (E > kMaxExperts || !small_tiles || !big_tiles || big_m < 1 ||
        (split_small && P > kSmallPairs))
        return hipErrorInvalidValue;
    const TileOut t{small_max, big_m, split_small ? 1 : 0, small_tiles, num_small, big_tiles,
                    num_big};
    return permute_impl(P, E, ids, counts, offsets, row_to_pair, pair_to_row, chunk_scratch, t,
                        s);
}

hipError_t launch_build_tiles(const int32_t* offsets, int32_t E, int32_t small_max,
                              int32_t big_m, Tile* small_tiles, int32_t* num_small,
                              Tile* big_tiles, int32_t* num_big, hipStream_t s) {
    build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, small_max, big_m, small_tiles, num_small,
                                          big_tiles, num_big);
    return hipGetLastError();
}

}  // namespace moe
