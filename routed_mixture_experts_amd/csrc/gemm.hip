// Grouped and dense GEMMs of the routed-MoE forward on gfx950.
//
// The expert MLP is grouped matmul gate/up -> activation -> grouped matmul
// down ("vLLM-Ascend Kimi K3 MoE Forward Insight", Stage 4); the router
// product, the latent down-projection, the shared expert and the tail
// up-projection ("vllm.models.kimi_k3.nvidia.latent_moe_runner",
// _fused_forward, _overlap_allreduce_tail / _shard_up_proj_tail) are the same
// "NT" product with one group.  Every product here is
//     C[r, n] = sum_k A[arow(r), k] * B_g[n, k]  (+ a second K segment),
// both operands K-contiguous, with the epilogue fused (fp32 store, fp32 + bias
// row, layer-dtype store, or SwiGLU silu(gate) * up).
//
// Kernels:
//  * gemm_bf16_big    -- 256x256 tiles, 8 waves, a 4-slot LDS ring filled by
//    global_load_lds and operand fragments pipelined one K stage ahead: groups
//    with more than 64 rows (prefill) and large dense products.
//  * gemm_bf16_tiled  -- 128x128x64 LDS double-buffered tiles, 4 waves in a
//    2x2 layout, each wave a 64x64 block of v_mfma_f32_32x32x16_bf16: mid-size
//    dense products.
//  * gemm_bf16_stream -- groups of at most 64 rows (all of decode): the weights
//    are the streamed operand.  Each wave of an 8-wave workgroup streams 16
//    whole weight rows straight into MFMA registers; the token rows come from
//    an LDS double buffer.
//  * gemm_bf16_stream_ksplit -- the same product with K split over 4 waves, for
//    dense products too small to fill the chip with whole-row streams.
//  * gemm_f32_tiled   -- fp32 VALU 64x64 tiles for the fp32 layer.
// Work is a flat list of (row tile, column tile); workgroup i runs on XCD
// i % 8, so logical tile ids are remapped to give each XCD a contiguous range,
// taken in bands of row tiles so that the workgroups resident on one XCD share
// both operands' K slices in its L2.
#include "common.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int xcd_remap(int i, int total) {
    const int xcd = i & 7, local = i >> 3;
    const int per = total >> 3, rem = total & 7;
    return xcd * per + min(xcd, rem) + local;
}

struct TileCoord {
    int group, row0, row1, nt;
};

// Row tiles per band in the launch order of one group's tiles.
constexpr int kBandRows = 4;

// Position o of a block of cnt row tiles x ntn column tiles, taken in bands of
// kBandRows row tiles; inside a band the row tile varies fastest, so the
// workgroups resident on one XCD at a time form a kBandRows x (32 /
// kBandRows) block and reuse both operands' K slices from its L2.
__device__ __forceinline__ void band_order(int o, int cnt, int ntn, int& mt, int& nt) {
    const int band = o / (kBandRows * ntn);
    const int in_band = o - band * kBandRows * ntn;
    const int rows = min(kBandRows, cnt - band * kBandRows);
    nt = in_band / rows;
    mt = band * kBandRows + (in_band - nt * rows);
}

// Returns false when this workgroup has no tile (grids are sized from an
// upper bound of the tile count).
__device__ __forceinline__ bool fetch_tile(const GemmArgs& g, int tile_m, int ntn, TileCoord& c) {
    const int nm = g.tiles ? *g.num_tiles : (g.M + tile_m - 1) / tile_m;
    const int total = nm * ntn;
    const int i = blockIdx.x;
    if (i >= total) return false;
    const int lid = xcd_remap(i, total);
    int mt;
    if (g.tiles) {
        // the tiles of one group are contiguous: tile lid / ntn belongs to the
        // group whose block of count * ntn workgroups holds lid
        const Tile t0 = g.tiles[lid / ntn];
        const int first = __builtin_amdgcn_readfirstlane(t0.first);
        const int cnt = __builtin_amdgcn_readfirstlane(t0.count);
        band_order(lid - first * ntn, cnt, ntn, mt, c.nt);
        const Tile t = g.tiles[first + mt];
        // the tile is the same for the whole workgroup: keep it in SGPRs so
        // that every branch on it is a scalar branch
        c.group = __builtin_amdgcn_readfirstlane(t.group);
        c.row0 = __builtin_amdgcn_readfirstlane(t.row0);
        c.row1 = __builtin_amdgcn_readfirstlane(t.row1);
    } else {
        band_order(lid, nm, ntn, mt, c.nt);
        c.group = 0;
        c.row0 = mt * tile_m;
        c.row1 = min(c.row0 + tile_m, g.M);
    }
    return true;
}

__device__ __forceinline__ int64_t a_row_of(const GemmArgs& g, int r) {
    return g.a_map ? (int64_t)(g.a_map[r] / g.a_div) : (int64_t)r;
}

// ------------------------------------------------------------------------
// bf16 LDS-tiled MFMA kernel
// ------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TBK = 64, TLD = TBK + 8;  // LDS row stride (elements)

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_tiled(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + 63) / 64 : (g.N + TBN - 1) / TBN;
    TileCoord tc;
    if (!fetch_tile(g, TBM, ntn, tc)) return;

    __shared__ __attribute__((aligned(16))) bf16_t smem[2][2][TBM * TLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = tid >> 3, lcol = (tid & 7) * 8;

    const bf16_t* A = (const bf16_t*)g.A;
    const bf16_t* Bg = (const bf16_t*)g.B + (int64_t)tc.group * g.b_gstride;
    const bf16_t* A2 = (const bf16_t*)g.A2;
    const bf16_t* B2 = (const bf16_t*)g.B2;

    const bf16_t* ap[4];
    const bf16_t* bp[4];
    const bf16_t* ap2[4];
    const bf16_t* bp2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = min(tc.row0 + lrow + 32 * i, tc.row1 - 1);
        ap[i] = A + a_row_of(g, rr) * g.lda + lcol;
        ap2[i] = A2 ? A2 + (int64_t)rr * g.lda2 + lcol : nullptr;
        const int rho = lrow + 32 * i;
        int wrow;
        if (SW) {
            const int c = min(tc.nt * 64 + (rho & 63), g.N - 1);
            wrow = rho < 64 ? c : g.N + c;
        } else {
            wrow = min(tc.nt * TBN + rho, g.N - 1);
        }
        bp[i] = Bg + (int64_t)wrow * g.K + lcol;
        bp2[i] = B2 ? B2 + (int64_t)wrow * g.K2 + lcol : nullptr;
    }

    const int nk1 = g.K / TBK;
    const int nk = nk1 + (A2 ? g.K2 / TBK : 0);

    u32x4_t ra[4], rb[4];
    auto gload = [&](int kt) {
        if (kt < nk1) {
            const int ko = kt * TBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *(const u32x4_t*)(ap[i] + ko);
                rb[i] = *(const u32x4_t*)(bp[i] + ko);
            }
        } else {
            const int ko = (kt - nk1) * TBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *(const u32x4_t*)(ap2[i] + ko);
                rb[i] = *(const u32x4_t*)(bp2[i] + ko);
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4_t*)(&smem[buf][0][(lrow + 32 * i) * TLD + lcol]) = ra[i];
            *(u32x4_t*)(&smem[buf][1][(lrow + 32 * i) * TLD + lcol]) = rb[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][nj][j] = 0.0f;

    const int fr = lane & 31, fk = (lane >> 5) * 8;
    int brow[2];
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) brow[nj] = SW ? (nj * 64 + wn * 32) : (wn * 64 + nj * 32);

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const bf16_t* sa = smem[buf][0];
        const bf16_t* sb = smem[buf][1];
#pragma unroll
        for (int kk = 0; kk < TBK / 16; ++kk) {
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                fa[mi] = *(const bf16x8_t*)(&sa[(wm * 64 + mi * 32 + fr) * TLD + kk * 16 + fk]);
#pragma unroll
            for (int nj = 0; nj < 2; ++nj)
                fb[nj] = *(const bf16x8_t*)(&sb[(brow[nj] + fr) * TLD + kk * 16 + fk]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int nj = 0; nj < 2; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[nj],
                                                                           acc[mi][nj], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds column fr of each 32x32 block, rows 8*(j/4)+4*(lane/32)+j%4
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = tc.row0 + wm * 64 + mi * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            if (r >= tc.row1) continue;
            if (SW) {
                const int hc = tc.nt * 64 + wn * 32 + fr;
                if (hc < g.N) {
                    const float h = silu_f32(acc[mi][0][j]) * acc[mi][1][j];
                    ((bf16_t*)g.C)[(int64_t)r * g.ldc + hc] = f32_to_bf16(h);
                }
            } else {
#pragma unroll
                for (int nj = 0; nj < 2; ++nj) {
                    const int c = tc.nt * TBN + wn * 64 + nj * 32 + fr;
                    if (c >= g.N) continue;
                    float v = acc[mi][nj][j];
                    if (EPI == EPI_F32_BIAS && g.bias) v += g.bias[c];
                    if (EPI == EPI_OUT)
                        ((bf16_t*)g.C)[(int64_t)r * g.ldc + c] = f32_to_bf16(v);
                    else
                        ((float*)g.C)[(int64_t)r * g.ldc + c] = v;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// bf16 256x256 MFMA kernel for grouped products with many rows per group
// ------------------------------------------------------------------------
// 8 waves (two per SIMD) in a 2x4 layout; each wave owns a 128x64 block of
// 4x2 v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators per lane).  K
// advances 64 at a time through a 2-slot LDS ring (64 KB per stage) filled
// directly from global memory by global_load_lds_dwordx4.  Each DMA
// instruction moves 8 rows x 128 bytes, whole cache lines: with 16 rows x 64
// bytes per instruction the L2-to-LDS path delivers 2.4x less (measured 12.5
// against 30 TB/s on L2-resident tiles).  LDS row r (128 bytes) keeps its
// eight 16-byte chunks at chunk ^ ((r & 7) ^ ((r >> 3) & 1)), so the MFMA
// operand reads (32 rows, one chunk) hit distinct banks for any 8
// consecutive rows and, per row parity, any 16; a lane therefore fetches the
// global chunk whose swizzled slot is its own.  Operand fragments are read
// half a stage ahead of their MFMAs: while stage kt's first half is
// multiplied, its second half is read; then one barrier publishes stage kt+1
// (its DMA was issued a whole stage earlier) and frees stage kt's slot for
// the DMA of stage kt+2; while stage kt's second half is multiplied, stage
// kt+1's first half is read.  A wave whose 128 rows all lie past the tile's
// end skips its MFMAs.
constexpr int GBM = 256, GBN = 256, GBK = 64, GSLOTS = 2;

__device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

// s_waitcnt with only a vector-memory count (gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same with lgkmcnt(0) as well.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

template <int EPI, bool KCAT>
__global__ __launch_bounds__(512, 1) void gemm_bf16_big(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + 127) / 128 : (g.N + GBN - 1) / GBN;
    TileCoord tc;
    if (!fetch_tile(g, GBM, ntn, tc)) return;

    // one LDS buffer: ring slot s holds the A tile at [s][0] and the B tile at
    // [s][1]; after the K loop the epilogue reuses it as a flat fp32 buffer
    __shared__ __attribute__((aligned(1024))) bf16_t smem[GSLOTS][2][GBM * GBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    const bf16_t* Bg = (const bf16_t*)g.B + (int64_t)tc.group * g.b_gstride;
    const char* Ab = (const char*)g.A;
    const char* Bb = (const char*)Bg;
    const char* A2b = (const char*)g.A2;
    const char* B2b = (const char*)g.B2;

    // DMA block i of this wave covers tile rows 32*wave + 8*i .. +7 of A and
    // of B; lane l fills row +l/8, slot l%8, i.e. global chunk
    // (l%8) ^ swizzle(row).  The swizzle reads bits 0..3 of the row: l/8 and
    // the parity of i.  32-bit byte offsets from wave-uniform bases; rows past
    // the tile's end load the tile's first row (never stored).
    uint32_t ao[4], bo[4], ao2[KCAT ? 4 : 1], bo2[KCAT ? 4 : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * wave + 8 * i + (lane >> 3);
        const int chunk_bytes = swz(row, lane & 7) * 16;
        const int r = tc.row0 + row;
        const int rr = r < tc.row1 ? r : tc.row0;
        ao[i] = (uint32_t)(a_row_of(g, rr) * g.lda * 2) + chunk_bytes;
        int wrow;
        if (SW) {
            const int c = min(tc.nt * 128 + (row & 127), g.N - 1);
            wrow = row < 128 ? c : g.N + c;
        } else {
            wrow = min(tc.nt * GBN + row, g.N - 1);
        }
        bo[i] = (uint32_t)((int64_t)wrow * g.K * 2) + chunk_bytes;
        if (KCAT) {
            ao2[i] = (uint32_t)((int64_t)rr * g.lda2 * 2) + chunk_bytes;
            bo2[i] = (uint32_t)((int64_t)wrow * g.K2 * 2) + chunk_bytes;
        }
    }

    const int nk1 = g.K / GBK;
    const int nk = nk1 + (KCAT ? g.K2 / GBK : 0);

    // Issue stage kt (clamped to the last stage) into its ring slot: 8 DMA
    // instructions per wave.  The K segment of a K-concatenated product is
    // picked with selects.
    auto issue = [&](int kt) __attribute__((always_inline)) {
        const int slot = kt & (GSLOTS - 1);
        kt = min(kt, nk - 1);
        const bool seg1 = !KCAT || kt < nk1;
        const char* abase = seg1 ? Ab : A2b;
        const char* bbase = seg1 ? Bb : B2b;
        const uint32_t ko = (uint32_t)(seg1 ? kt : kt - nk1) * GBK * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = (32 * wave + 8 * i) * GBK;
            __builtin_amdgcn_global_load_lds(
                (const void*)(abase + ((seg1 ? ao[i] : ao2[KCAT ? i : 0]) + ko)),
                (lds_ptr_t)&smem[slot][0][blk], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const void*)(bbase + ((seg1 ? bo[i] : bo2[KCAT ? i : 0]) + ko)),
                (lds_ptr_t)&smem[slot][1][blk], 16, 0, 0);
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][nj][j] = 0.0f;

    // Operand fragments of v_mfma_f32_32x32x16_bf16: lane (fr, fh) supplies
    // row fr, k 8*fh .. +7 of 16-deep step ks, i.e. LDS chunk 2*ks + fh.
    const int fr = lane & 31, fh = lane >> 5;
    int aoffs[4][4], boffs[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int ch = ks * 2 + fh;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int row = wm * 128 + mi * 32 + fr;
            aoffs[ks][mi] = row * GBK + swz(row, ch) * 8;
        }
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            const int row = (SW ? nj * 128 + wn * 32 : wn * 64 + nj * 32) + fr;
            boffs[ks][nj] = row * GBK + swz(row, ch) * 8;
        }
    }

    // does this wave's 128-row half hold any row of the tile (wave-uniform)
    const bool active = tc.row1 - tc.row0 > wm * 128;

    // Fragments of one half stage (two 16-deep steps).
    struct Frags {
        bf16x8_t a[2][4], b[2][2];
    };
    auto read_half = [&](int kt, int h, Frags& f) __attribute__((always_inline)) {
        const bf16_t* a = smem[kt & (GSLOTS - 1)][0];
        const bf16_t* b = smem[kt & (GSLOTS - 1)][1];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int ks = 2 * h + s2;
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) f.b[s2][nj] = *(const bf16x8_t*)(&b[boffs[ks][nj]]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) f.a[s2][mi] = *(const bf16x8_t*)(&a[aoffs[ks][mi]]);
        }
    };
    auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int nj = 0; nj < 2; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        f.a[s2][mi], f.b[s2][nj], acc[mi][nj], 0, 0, 0);
    };

    issue(0);
    issue(1);
    wait_vmcnt_lgkm0<8>();  // this wave's part of stage 0 has landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Frags f0, f1;
    if (active) read_half(0, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
        if (active) {
            read_half(kt, 1, f1);
            mma(f0);
        }
        asm volatile("" ::: "memory");
        // stage kt+1's DMA (issued a stage ago) has landed for this wave and
        // its reads of stage kt are retired; after the barrier stage kt+1 is
        // visible everywhere and stage kt's slot takes stage kt+2
        wait_vmcnt_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(kt + 2);
        if (active) {
            read_half(kt + 1, 0, f0);
            mma(f1);
        }
        asm volatile("" ::: "memory");
    }
    // The ring's trailing DMAs must land before the LDS is reused below.
    wait_vmcnt<0>();
    __syncthreads();

    // Epilogue through LDS, one 32-row block of each wave at a time: the
    // accumulators are written in MFMA layout (lane = column, 16 rows), then
    // each lane reads back half a row and stores it with 16-byte writes.  Only
    // one block's accumulators are live in VGPRs at a time.  Row stride 72
    // floats keeps the writes free of bank
    // write conflicts (reads see at most two-way ones).  Each wave uses its
    // own region, so LDS order within the wave suffices between the writes and
    // the reads.
    if (!active) return;
    constexpr int ELD = 72;
    float* ep = (float*)&smem[0][0][0] + wave * 32 * ELD;
    const int er = lane >> 1, eh = lane & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                ep[(8 * (j >> 2) + 4 * fh + (j & 3)) * ELD + nj * 32 + fr] = acc[mi][nj][j];
        asm volatile("" ::: "memory");
        const int r = tc.row0 + wm * 128 + mi * 32 + er;
        const float* src = ep + er * ELD;
        if (r < tc.row1) {
            if (SW) {
                // columns 0..31 of the wave block are gate, 32..63 up, for the
                // wave's 32 h columns; this lane takes 16 of them
                const int hc0 = tc.nt * 128 + wn * 32 + eh * 16;
                bf16_t* dst = (bf16_t*)g.C + (int64_t)r * g.ldc + hc0;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const f32x4_t g0 = *(const f32x4_t*)(src + eh * 16 + q * 8);
                    const f32x4_t g1 = *(const f32x4_t*)(src + eh * 16 + q * 8 + 4);
                    const f32x4_t u0 = *(const f32x4_t*)(src + 32 + eh * 16 + q * 8);
                    const f32x4_t u1 = *(const f32x4_t*)(src + 32 + eh * 16 + q * 8 + 4);
                    u32x4_t o;
                    o[0] = pack_bf16x2(silu_f32(g0[0]) * u0[0], silu_f32(g0[1]) * u0[1]);
                    o[1] = pack_bf16x2(silu_f32(g0[2]) * u0[2], silu_f32(g0[3]) * u0[3]);
                    o[2] = pack_bf16x2(silu_f32(g1[0]) * u1[0], silu_f32(g1[1]) * u1[1]);
                    o[3] = pack_bf16x2(silu_f32(g1[2]) * u1[2], silu_f32(g1[3]) * u1[3]);
                    if (hc0 + q * 8 < g.N) *(u32x4_t*)(dst + q * 8) = o;
                }
            } else {
                const int c0 = tc.nt * GBN + wn * 64 + eh * 32;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = c0 + q * 8;
                    if (c >= g.N) continue;
                    f32x4_t v0 = *(const f32x4_t*)(src + eh * 32 + q * 8);
                    f32x4_t v1 = *(const f32x4_t*)(src + eh * 32 + q * 8 + 4);
                    if (EPI == EPI_F32_BIAS && g.bias) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            v0[t] += g.bias[c + t];
                            v1[t] += g.bias[c + 4 + t];
                        }
                    }
                    if (EPI == EPI_OUT) {
                        u32x4_t o;
                        o[0] = pack_bf16x2(v0[0], v0[1]);
                        o[1] = pack_bf16x2(v0[2], v0[3]);
                        o[2] = pack_bf16x2(v1[0], v1[1]);
                        o[3] = pack_bf16x2(v1[2], v1[3]);
                        *(u32x4_t*)((bf16_t*)g.C + (int64_t)r * g.ldc + c) = o;
                    } else {
                        float* dst = (float*)g.C + (int64_t)r * g.ldc + c;
                        *(f32x4_t*)dst = v0;
                        *(f32x4_t*)(dst + 4) = v1;
                    }
                }
            }
        }
        asm volatile("" ::: "memory");
    }
}

// ------------------------------------------------------------------------
// bf16 weight-streaming MFMA kernel (<= 64 rows per tile)
// ------------------------------------------------------------------------
constexpr int SROWS = 16;   // token rows per MFMA block (and per dense tile)
constexpr int SNW = 64;     // weight rows per workgroup

// One tile of up to 16*NB token rows: each wave streams its quarter of K for
// 64 weight rows and applies every weight fragment to all NB token blocks.
// SU k-steps (of 32) form one load batch; two batches are in flight.
template <int EPI, int NB, int SU>
__device__ __forceinline__ void stream_tile(const GemmArgs& g, const TileCoord& tc,
                                            float (*red)[4][4][64]) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kofs = (lane >> 4) * 8;

    // 32-bit byte offsets from wave-uniform bases (one VGPR per row); every
    // operand of one group fits in 4 GiB (checked on the host)
    const char* Bb = (const char*)((const bf16_t*)g.B + (int64_t)tc.group * g.b_gstride);
    const char* B2b = (const char*)g.B2;
    const char* Ab = (const char*)g.A;
    const char* A2b = (const char*)g.A2;
    uint32_t wo[4], wo2[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int wrow;
        if (SW) {
            const int c = min(tc.nt * 32 + (q & 1) * 16 + l16, g.N - 1);
            wrow = q < 2 ? c : g.N + c;
        } else {
            wrow = min(tc.nt * SNW + q * 16 + l16, g.N - 1);
        }
        wo[q] = (uint32_t)((int64_t)wrow * g.K * 2) + kofs * 2;
        wo2[q] = (uint32_t)((int64_t)wrow * g.K2 * 2) + kofs * 2;
    }
    uint32_t xo[NB], xo2[NB];
    bool xvalid[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        const int r = tc.row0 + tb * 16 + l16;
        xvalid[tb] = r < tc.row1;
        xo[tb] = (uint32_t)((xvalid[tb] ? a_row_of(g, r) : 0) * g.lda * 2) + kofs * 2;
        xo2[tb] = (uint32_t)((int64_t)(xvalid[tb] ? r : 0) * g.lda2 * 2) + kofs * 2;
    }

    const int ns1 = g.K / 32;
    const int ns = ns1 + (g.A2 ? g.K2 / 32 : 0);
    const int s0 = (int)((int64_t)wave * ns / 4), s1 = (int)((int64_t)(wave + 1) * ns / 4);

    f32x4_t acc[4][NB];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) acc[q][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wa[SU][4], xa[SU][NB], wb[SU][4], xb[SU][NB];
    const u32x4_t zero = {0u, 0u, 0u, 0u};

    auto load = [&](int sbase, u32x4_t (&w)[SU][4], u32x4_t (&x)[SU][NB])
                    __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int st = sbase + u;
            if (st < s1) {
                if (st < ns1) {
                    const uint32_t ko = st * 64;
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[u][q] = *(const u32x4_t*)(Bb + (wo[q] + ko));
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb)
                        x[u][tb] = xvalid[tb] ? *(const u32x4_t*)(Ab + (xo[tb] + ko)) : zero;
                } else {
                    const uint32_t ko = (st - ns1) * 64;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[u][q] = *(const u32x4_t*)(B2b + (wo2[q] + ko));
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb)
                        x[u][tb] = xvalid[tb] ? *(const u32x4_t*)(A2b + (xo2[tb] + ko)) : zero;
                }
            }
        }
    };
    auto compute = [&](int sbase, u32x4_t (&w)[SU][4], u32x4_t (&x)[SU][NB])
                       __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            if (sbase + u < s1) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const bf16x8_t xb8 = __builtin_bit_cast(bf16x8_t, x[u][tb]);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[q][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, w[u][q]), xb8, acc[q][tb], 0, 0, 0);
                }
            }
        }
    };

    load(s0, wa, xa);
    for (int s = s0; s < s1; s += 2 * SU) {
        load(s + SU, wb, xb);
        compute(s, wa, xa);
        load(s + 2 * SU, wa, xa);
        compute(s + SU, wb, xb);
    }

    // acc[q][tb][j] holds C[weight row 4*(lane/16)+j of group q][token 16*tb + lane%16]
    const int wr = (lane >> 4) * 4;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        if (tb > 0) __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wave][q][j][lane] = acc[q][tb][j];
        __syncthreads();
        const int rr = tc.row0 + tb * 16 + l16;
        if (SW) {
            if (wave < 2) {
                const int q = wave;
                float gsum[4], usum[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gsum[j] = red[0][q][j][lane] + red[1][q][j][lane] + red[2][q][j][lane] +
                              red[3][q][j][lane];
                    usum[j] = red[0][q + 2][j][lane] + red[1][q + 2][j][lane] +
                              red[2][q + 2][j][lane] + red[3][q + 2][j][lane];
                }
                if (rr < tc.row1) {
                    bf16_t* crow = (bf16_t*)g.C + (int64_t)rr * g.ldc;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int hc = tc.nt * 32 + q * 16 + wr + j;
                        if (hc < g.N) crow[hc] = f32_to_bf16(silu_f32(gsum[j]) * usum[j]);
                    }
                }
            }
        } else {
            const int q = wave;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = red[0][q][j][lane] + red[1][q][j][lane] + red[2][q][j][lane] +
                       red[3][q][j][lane];
            if (rr < tc.row1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = tc.nt * SNW + q * 16 + wr + j;
                    if (c >= g.N) continue;
                    float o = v[j];
                    if (EPI == EPI_F32_BIAS && g.bias) o += g.bias[c];
                    if (EPI == EPI_OUT)
                        ((bf16_t*)g.C)[(int64_t)rr * g.ldc + c] = f32_to_bf16(o);
                    else
                        ((float*)g.C)[(int64_t)rr * g.ldc + c] = o;
                }
            }
        }
    }
}

// Dense products with few tiles: splitting K over the waves keeps more of
// the chip busy than whole-row streams would.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_stream_ksplit(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + 31) / 32 : (g.N + SNW - 1) / SNW;
    TileCoord tc;
    if (!fetch_tile(g, SROWS, ntn, tc)) return;
    __shared__ float red[4][4][4][64];
    const int rows = tc.row1 - tc.row0;
    if (rows <= 16) stream_tile<EPI, 1, 4>(g, tc, red);
    else if (rows <= 32) stream_tile<EPI, 2, 2>(g, tc, red);
    else stream_tile<EPI, 4, 2>(g, tc, red);
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt left at "no wait").
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Whole-row weight streams.  Each wave owns 16 weight rows (SwiGLU: 8 gate
// rows and the 8 up rows of the same hidden columns) over the full K, so
// every wave reads 16 long contiguous rows -- the pattern that keeps HBM
// near its streaming rate; splitting K over waves (four read positions per
// row) runs about 12% slower.  The token rows, shared by the 4 waves, come
// from LDS: chunks of CS k-steps are loaded a chunk ahead into registers
// (each wave a quarter of the chunk), written to a double buffer, and
// published with one barrier per chunk.  Weight fragments run PD k-steps
// ahead in registers.  Reading the token operand straight from global
// memory beside the weights costs up to a third of the bandwidth, which is
// why it is staged.  Every vector-memory operation here is a register load,
// so the compiler's in-order vmcnt bookkeeping stays exact (LDS-DMA loads
// mixed with register loads make it fall back to draining the counter).
constexpr int SX_BYTES = 64 * 1024;  // token-chunk double buffer
constexpr int SRW = 8;               // waves per workgroup
constexpr int SRN = 16 * SRW;        // weight rows per workgroup (SwiGLU: SRN / 2 columns)

template <int EPI, int NB, bool KCAT>
__device__ __forceinline__ void stream_rows_tile(const GemmArgs& g, const TileCoord& tc,
                                                 char* xs) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr int CS = NB == 4 ? 8 : 16;   // k-steps (of 32) per token chunk
    constexpr int PD = 8;                  // weight prefetch distance in k-steps
    constexpr int XI = CS * NB / SRW;      // 1 KB token blocks per wave per chunk
    constexpr int CHUNK = CS * NB * 1024;  // bytes of one token chunk
    static_assert(2 * CHUNK <= SX_BYTES && CS % PD == 0 && XI % NB == 0, "stream tiling");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;

    // 32-bit byte offsets from wave-uniform bases; every operand of one group
    // fits in 4 GiB (checked on the host)
    const char* Bb = (const char*)((const bf16_t*)g.B + (int64_t)tc.group * g.b_gstride);
    const char* B2b = (const char*)g.B2;
    const char* Ab = (const char*)g.A;
    const char* A2b = (const char*)g.A2;
    int wrow;
    if (SW) {
        const int c = min(tc.nt * (SRN / 2) + wave * 8 + (l16 & 7), g.N - 1);
        wrow = l16 < 8 ? c : g.N + c;
    } else {
        wrow = min(tc.nt * SRN + wave * 16 + l16, g.N - 1);
    }
    const uint32_t wo = (uint32_t)((int64_t)wrow * g.K * 2) + g4 * 16;
    const uint32_t wo2 = KCAT ? (uint32_t)((int64_t)wrow * g.K2 * 2) + g4 * 16 : 0u;
    // token rows past the tile's end load its last row (never stored)
    uint32_t xo[NB], xo2[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        const int r = min(tc.row0 + tb * 16 + l16, tc.row1 - 1);
        xo[tb] = (uint32_t)(a_row_of(g, r) * g.lda * 2) + g4 * 16;
        xo2[tb] = KCAT ? (uint32_t)((int64_t)r * g.lda2 * 2) + g4 * 16 : 0u;
    }

    const int ns1 = g.K / 32;
    const int ns = ns1 + (KCAT ? g.K2 / 32 : 0);
    const int nch = (ns + CS - 1) / CS;

    // Token chunk c lives in LDS buffer c & 1 as 1 KB blocks b = (k-step
    // b / NB, 16-row block b % NB), each in MFMA operand order (lane l holds
    // row l % 16, k 8 * (l / 16) .. +7 of the step).  This wave moves blocks
    // wave * XI .. +XI-1; steps past K re-read the last step (never used).
    u32x4_t xr[XI];
    auto load_x = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int b = wave * XI + i;
            const int tb = i % NB;
            const int st = min(c * CS + b / NB, ns - 1);
            const bool seg1 = !KCAT || st < ns1;
            const char* src = seg1 ? Ab + (xo[tb] + (uint32_t)st * 64)
                                   : A2b + (xo2[tb] + (uint32_t)(st - ns1) * 64);
            xr[i] = *(const u32x4_t*)src;
        }
    };
    auto store_x = [&](int c) __attribute__((always_inline)) {
        char* dst = xs + (c & 1) * CHUNK + lane * 16;
#pragma unroll
        for (int i = 0; i < XI; ++i) *(u32x4_t*)(dst + (wave * XI + i) * 1024) = xr[i];
    };
    auto load_w = [&](int st) __attribute__((always_inline)) {
        st = min(st, ns - 1);
        const bool seg1 = !KCAT || st < ns1;
        const char* src = seg1 ? Bb + (wo + (uint32_t)st * 64) : B2b + (wo2 + (uint32_t)(st - ns1) * 64);
        return *(const u32x4_t*)src;
    };

    f32x4_t acc[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t w[PD];

    // The first weight fragments go out before the wait for chunk 0.  Order
    // is pinned (empty asm with a memory clobber) so that on both paths into
    // the store of chunk c + 1 the token loads are followed by exactly the CS
    // weight loads of chunk c: the compiler's wait for the token registers
    // then leaves the newest weight loads in flight.
    load_x(0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int v = 0; v < PD; ++v) w[v] = load_w(v);
    asm volatile("" ::: "memory");
    store_x(0);
    asm volatile("" ::: "memory");
    load_x(1);
    asm volatile("" ::: "memory");

    for (int c = 0; c < nch; ++c) {
        // this wave's LDS writes of chunk c are done, and its LDS reads of
        // chunk c - 1; after the barrier every wave's part of chunk c is
        // visible and no wave reads buffer (c + 1) & 1 any more.  (A
        // __syncthreads fence would also drain the weight loads in flight.)
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const char* xc = xs + (c & 1) * CHUNK + lane * 16;
#pragma unroll
        for (int u = 0; u < CS; u += PD) {
#pragma unroll
            for (int v = 0; v < PD; ++v) {
                // steps past K (the ragged last chunk) multiply zero weights
                const int st = c * CS + u + v;
                const u32x4_t wz = st < ns ? w[v] : u32x4_t{0u, 0u, 0u, 0u};
                const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, wz);
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const u32x4_t xv = *(const u32x4_t*)(xc + ((u + v) * NB + tb) * 1024);
                    acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        wf, __builtin_bit_cast(bf16x8_t, xv), acc[tb], 0, 0, 0);
                }
                w[v] = load_w(st + PD);
            }
        }
        asm volatile("" ::: "memory");
        // chunk c + 1 has had a whole chunk to arrive; chunks past the end
        // only touch the idle buffer, which keeps this branch-free
        store_x(c + 1);
        asm volatile("" ::: "memory");
        load_x(c + 2);
        asm volatile("" ::: "memory");
    }

    // acc[tb][j] = C[weight row 4*g4 + j of this wave][token 16*tb + l16]
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        const int r = tc.row0 + tb * 16 + l16;
        if (SW) {
            // lanes 32..63 hold the up rows of lane - 32's gate rows
            float up[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) up[j] = __shfl_xor(acc[tb][j], 32);
            if (g4 < 2 && r < tc.row1) {
                bf16_t* crow = (bf16_t*)g.C + (int64_t)r * g.ldc;
                const int hc0 = tc.nt * (SRN / 2) + wave * 8 + g4 * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (hc0 + j < g.N) crow[hc0 + j] = f32_to_bf16(silu_f32(acc[tb][j]) * up[j]);
            }
        } else if (r < tc.row1) {
            const int c0 = tc.nt * SRN + wave * 16 + g4 * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = c0 + j;
                if (c >= g.N) continue;
                float o = acc[tb][j];
                if (EPI == EPI_F32_BIAS && g.bias) o += g.bias[c];
                if (EPI == EPI_OUT)
                    ((bf16_t*)g.C)[(int64_t)r * g.ldc + c] = f32_to_bf16(o);
                else
                    ((float*)g.C)[(int64_t)r * g.ldc + c] = o;
            }
        }
    }
}

// Grouped tiles here hold one whole group of at most 64 rows; dense products
// are cut into 16-row tiles.
template <int EPI, bool KCAT>
__global__ __launch_bounds__(64 * SRW, 4) void gemm_bf16_stream(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + SRN / 2 - 1) / (SRN / 2) : (g.N + SRN - 1) / SRN;
    TileCoord tc;
    if (!fetch_tile(g, SROWS, ntn, tc)) return;
    __shared__ __attribute__((aligned(1024))) char xs[SX_BYTES];
    const int rows = tc.row1 - tc.row0;
    if (rows <= 16) stream_rows_tile<EPI, 1, KCAT>(g, tc, xs);
    else if (rows <= 32) stream_rows_tile<EPI, 2, KCAT>(g, tc, xs);
    else stream_rows_tile<EPI, 4, KCAT>(g, tc, xs);
}

// ------------------------------------------------------------------------
// fp32 VALU tiled kernel (64x64 tiles, 4x4 outputs per thread)
// ------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_tiled(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + 31) / 32 : (g.N + FBN - 1) / FBN;
    TileCoord tc;
    if (!fetch_tile(g, FBM, ntn, tc)) return;

    __shared__ float As[FBK][FBM + 4];
    __shared__ float Bs[FBK][FBN + 4];

    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int lr = tid >> 2, lk = (tid & 3) * 4;

    const float* A = (const float*)g.A;
    const float* Bg = (const float*)g.B + (int64_t)tc.group * g.b_gstride;
    const int rr = min(tc.row0 + lr, tc.row1 - 1);
    const float* ap = A + a_row_of(g, rr) * g.lda + lk;
    const float* ap2 = g.A2 ? (const float*)g.A2 + (int64_t)rr * g.lda2 + lk : nullptr;
    int wrow;
    if (SW) {
        const int c = min(tc.nt * 32 + (lr & 31), g.N - 1);
        wrow = lr < 32 ? c : g.N + c;
    } else {
        wrow = min(tc.nt * FBN + lr, g.N - 1);
    }
    const float* bp = Bg + (int64_t)wrow * g.K + lk;
    const float* bp2 = g.B2 ? (const float*)g.B2 + (int64_t)wrow * g.K2 + lk : nullptr;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    int bcol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bcol[j] = SW ? (j < 2 ? tx * 2 + j : 32 + tx * 2 + j - 2) : tx * 4 + j;

    const int nk1 = g.K / FBK;
    const int nk = nk1 + (g.A2 ? g.K2 / FBK : 0);
    for (int kt = 0; kt < nk; ++kt) {
        f32x4_t av, bv;
        if (kt < nk1) {
            av = *(const f32x4_t*)(ap + kt * FBK);
            bv = *(const f32x4_t*)(bp + kt * FBK);
        } else {
            av = *(const f32x4_t*)(ap2 + (kt - nk1) * FBK);
            bv = *(const f32x4_t*)(bp2 + (kt - nk1) * FBK);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            As[lk + i][lr] = av[i];
            Bs[lk + i][lr] = bv[i];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < FBK; ++k) {
            float a4[4], b4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a4[i] = As[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b4[j] = Bs[k][bcol[j]];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a4[i], b4[j], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tc.row0 + ty * 4 + i;
        if (r >= tc.row1) continue;
        if (SW) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int hc = tc.nt * 32 + tx * 2 + j;
                if (hc < g.N) {
                    const float gt = acc[i][j], up = acc[i][j + 2];
                    ((float*)g.C)[(int64_t)r * g.ldc + hc] = gt / (1.0f + expf(-gt)) * up;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = tc.nt * FBN + tx * 4 + j;
                if (c >= g.N) continue;
                float v = acc[i][j];
                if (EPI == EPI_F32_BIAS && g.bias) v += g.bias[c];
                ((float*)g.C)[(int64_t)r * g.ldc + c] = v;
            }
        }
    }
}

template <bool KC>
void launch_big(const GemmArgs& g, dim3 gd, hipStream_t s) {
    const dim3 bd(512);
    switch (g.epi) {
        case EPI_F32: gemm_bf16_big<EPI_F32, KC><<<gd, bd, 0, s>>>(g); break;
        case EPI_F32_BIAS: gemm_bf16_big<EPI_F32_BIAS, KC><<<gd, bd, 0, s>>>(g); break;
        case EPI_OUT: gemm_bf16_big<EPI_OUT, KC><<<gd, bd, 0, s>>>(g); break;
        default: gemm_bf16_big<EPI_SWIGLU, KC><<<gd, bd, 0, s>>>(g); break;
    }
}

// Dense products with fewer workgroups than this split K over the waves.
constexpr int64_t kStreamRowsMinGrid = 1024;

template <bool KC>
void launch_stream_rows(const GemmArgs& g, dim3 gd, hipStream_t s) {
    const dim3 bd(64 * SRW);
    switch (g.epi) {
        case EPI_F32: gemm_bf16_stream<EPI_F32, KC><<<gd, bd, 0, s>>>(g); break;
        case EPI_F32_BIAS: gemm_bf16_stream<EPI_F32_BIAS, KC><<<gd, bd, 0, s>>>(g); break;
        case EPI_OUT: gemm_bf16_stream<EPI_OUT, KC><<<gd, bd, 0, s>>>(g); break;
        default: gemm_bf16_stream<EPI_SWIGLU, KC><<<gd, bd, 0, s>>>(g); break;
    }
}

int col_tiles(int path, int dtype, int epi, int N) {
    const bool sw = epi == EPI_SWIGLU;
    if (dtype == 0) return sw ? (N + 31) / 32 : (N + FBN - 1) / FBN;
    if (path == GEMM_STREAM) return sw ? (N + SRN / 2 - 1) / (SRN / 2) : (N + SRN - 1) / SRN;
    if (path == GEMM_BIG) return sw ? (N + 127) / 128 : (N + GBN - 1) / GBN;
    return sw ? (N + 63) / 64 : (N + TBN - 1) / TBN;
}

int row_tile(int path, int dtype) {
    if (dtype == 0) return FBM;
    if (path == GEMM_STREAM) return SROWS;
    return path == GEMM_BIG ? GBM : TBM;
}

}  // namespace

int gemm_row_tile(int dtype, int path) { return row_tile(path, dtype); }

hipError_t launch_gemm(int dtype, int path, const GemmArgs& g, hipStream_t s) {
    const int tm = row_tile(path, dtype);
    const int nm = g.tiles ? g.max_tiles : (g.M + tm - 1) / tm;
    const int64_t grid = (int64_t)nm * col_tiles(path, dtype, g.epi, g.N);
    if (grid <= 0) return hipSuccess;
    dim3 gd((unsigned)grid), bd(256);
#define MOE_GEMM_SWITCH(KERNEL)                                                   \
    switch (g.epi) {                                                              \
        case EPI_F32: KERNEL<EPI_F32><<<gd, bd, 0, s>>>(g); break;                \
        case EPI_F32_BIAS: KERNEL<EPI_F32_BIAS><<<gd, bd, 0, s>>>(g); break;      \
        case EPI_OUT: KERNEL<EPI_OUT><<<gd, bd, 0, s>>>(g); break;                \
        default: KERNEL<EPI_SWIGLU><<<gd, bd, 0, s>>>(g); break;                  \
    }
    if (dtype == 0) {
        MOE_GEMM_SWITCH(gemm_f32_tiled)
    } else if (path == GEMM_STREAM) {
        const bool sw = g.epi == EPI_SWIGLU;
        const int64_t grid_ks = (int64_t)nm * (sw ? (g.N + 31) / 32 : (g.N + SNW - 1) / SNW);
        if (!g.tiles && grid_ks < kStreamRowsMinGrid) {
            gd = dim3((unsigned)grid_ks);
            MOE_GEMM_SWITCH(gemm_bf16_stream_ksplit)
        } else if (g.A2) {
            launch_stream_rows<true>(g, gd, s);
        } else {
            launch_stream_rows<false>(g, gd, s);
        }
    } else if (path == GEMM_BIG) {
        if (g.A2) launch_big<true>(g, gd, s);
        else launch_big<false>(g, gd, s);
    } else {
        MOE_GEMM_SWITCH(gemm_bf16_tiled)
    }
#undef MOE_GEMM_SWITCH
    return hipGetLastError();
}

}  // namespace moe
