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
//  * gemm_bf16_big4   -- 256x256 tiles, 4 waves of 128x128, LDS rings of
//    64-deep K stages (2 A slots, 3 B slots) filled by global_load_lds,
//    fragments read one 16-deep step ahead; bf16, FP8 or MXFP4 weights (the
//    quantised ones converted at the fragment read): the large expert
//    groups (prefill) and large dense products, with or without a second K
//    segment.
//  * gemm_bf16_tiled  -- 128x128x64 LDS double-buffered tiles, 4 waves in a
//    2x2 layout, each wave a 64x64 block of v_mfma_f32_32x32x16_bf16: mid-size
//    dense products (bf16 weights).
//  * the weight-streaming kernels for groups of at most 64 rows (all of
//    decode) and small dense products live in gemm_stream.hip.
//  * gemm_f32_tiled   -- fp32 VALU 64x64 tiles for the fp32 layer.
// Work is a flat list of (row tile, column tile); workgroup i runs on XCD
// i % 8, so logical tile ids are remapped to give each XCD a contiguous range,
// taken in bands of row tiles so that the workgroups resident on one XCD share
// both operands' K slices in its L2.
#include "gemm_tiles.h"
#include "router.h"

#include <type_traits>

namespace moe {

namespace {

using namespace tiles;

// 8-byte LDS loads as a vector type (a struct type would drop the load's
// type-based alias information)
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------
// bf16 LDS-tiled MFMA kernel
// ------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TBK = 64, TLD = TBK + 8;  // LDS row stride (elements)

// Dense products only (one group, bf16 weights).
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
    // K slices (dense fp32 products, gridDim.y > 1): slice blockIdx.y takes
    // stages [kt0, kt1) and writes its partial sums to its own M x N block
    const int kt0 = (int)((int64_t)blockIdx.y * nk / gridDim.y);
    const int kt1 = (int)((int64_t)(blockIdx.y + 1) * nk / gridDim.y);
    float* cslice = (float*)g.C + (int64_t)blockIdx.y * g.M * g.ldc;

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

    gload(kt0);
    sstore(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
        const int buf = (kt - kt0) & 1;
        if (kt + 1 < kt1) gload(kt + 1);
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
        if (kt + 1 < kt1) sstore(buf ^ 1);
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
                    const float h = glu_f32(acc[mi][0][j], acc[mi][1][j], g);
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
                        cslice[(int64_t)r * g.ldc + c] = v;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// 256x256 MFMA kernel: groups with many rows per group, large dense products
// ------------------------------------------------------------------------
// 4 waves (one per SIMD) in a 2x2 layout; each wave owns a 128x128 block of
// 4x4 v_mfma_f32_32x32x16_bf16 tiles (256 fp32 accumulators per lane, kept
// in AGPRs).  K advances 64 at a time through two LDS rings, 2 slots of A
// (token) tiles and 3 of B (weight) tiles, filled directly from global
// memory by global_load_lds.  Each A DMA instruction moves 8 rows x 128
// bytes, whole cache lines: with 16 rows x 64 bytes per instruction the
// L2-to-LDS path delivers 2.4x less (measured 12.5 against 30 TB/s on
// L2-resident tiles).  LDS row r (128 bytes) keeps its eight 16-byte chunks
// at chunk ^ ((r & 7) ^ ((r >> 3) & 1)), so the MFMA operand reads (32 rows,
// one chunk) hit distinct banks for any 8 consecutive rows and, per row
// parity, any 16; a lane therefore fetches the global chunk whose swizzled
// slot is its own.  Per 16-deep step a wave reads 4 A and 4 B fragments for
// 16 MFMAs (a stage reads 128 KB of LDS); fragments are read one step ahead,
// and each step's reads and DMA instructions are placed one after each MFMA
// (scheduling fences), so that the one wave of a SIMD keeps its MFMA pipe
// fed; the stage's one barrier sits between its third and last steps.
//
// B slots by weight format:
//  * bf16: 128 bytes per weight row (32 KB), like A.
//  * FP8 (OCP e4m3 codes, one fp32 scale per weight row; grouped products
//    only): 64 bytes per row (16 KB), moved in 16 rows x 64 bytes per DMA
//    instruction; LDS row r keeps its four 16-byte chunks at chunk ^
//    ((r >> 2) & 3).  A fragment read takes a lane's 8 codes and turns them
//    into 8 bf16 values exactly; the row scales multiply the fp32 sums in
//    the epilogue.
//  * MXFP4 (OCP E2M1 codes, two per byte, one E8M0 exponent per 32 codes of
//    a row; grouped products only): 32 bytes per row (8 KB; LDS row r keeps
//    its two 16-byte chunks at chunk ^ ((r >> 3) & 1)), then one dword of
//    exponents per row, the 4 blocks holding the stage's 2.  A fragment read
//    takes a lane's 8 codes and its block exponent and turns them into 8
//    bf16 values, the scale applied by the conversion.
// bf16 products may carry a second K segment ([A | A2] . [B | B2]^T).
constexpr int GBM = 256, GBN = 256, GBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

__device__ __forceinline__ int swz8(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

template <int EPI, int WF, bool KCAT>
__global__ __launch_bounds__(256, 1) void gemm_bf16_big4(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr bool FP8 = WF == WF_FP8, FP4 = WF == WF_MXFP4;
    static_assert(!KCAT || WF == WF_BF16, "a second K segment: bf16 weights only");
    const int ntn = SW ? (g.N + 127) / 128 : (g.N + GBN - 1) / GBN;
    TileCoord tc;
    if (!fetch_tile(g, GBM, ntn, tc)) return;

    // B slot: bf16 rows (128 bytes per stage), FP8 codes (64 bytes), or MXFP4
    // codes (32 bytes) followed by one exponent dword per row
    constexpr int A_BYTES = GBM * GBK * 2;
    constexpr int B_ROW = FP8 ? GBK : FP4 ? GBK / 2 : GBK * 2;  // bytes per weight row
    constexpr int B_CODES = GBN * B_ROW;
    constexpr int B_BYTES = FP4 ? B_CODES + GBN * 4 : B_CODES;
    constexpr int AS = 2, BS = 3;
    constexpr int B_RING = AS * A_BYTES;
    static_assert(B_RING + BS * B_BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) char smem[B_RING + BS * B_BYTES];
    // DMA instructions per wave and stage (a wave's share is 64 rows): A 8
    // (8 rows x 128 B each); B 8 (bf16), 4 (FP8: 16 rows x 64 B), or 3
    // (MXFP4: 2 x 32 rows x 32 B of codes, 1 x 64 rows x 4 B of exponents)
    constexpr int NDA = 8, NDB = FP8 ? 4 : FP4 ? 3 : 8;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const char* Ab = (const char*)g.A;
    const char* Bb = (const char*)g.B + (FP4   ? (int64_t)tc.group * g.b_gstride / 2
                                         : FP8 ? (int64_t)tc.group * g.b_gstride
                                               : (int64_t)tc.group * g.b_gstride * 2);
    const char* Sb = FP4 ? (const char*)g.b_scale + (int64_t)tc.group * g.b_scale_gstride : nullptr;
    const char* A2b = (const char*)g.A2;
    const char* B2b = (const char*)g.B2;
    auto wrow_of = [&](int row) __attribute__((always_inline)) {
        if (SW) {
            const int c = min(tc.nt * 128 + (row & 127), g.N - 1);
            return row < 128 ? c : g.N + c;
        }
        return min(tc.nt * GBN + row, g.N - 1);
    };

    // A: lane l of DMA instruction i fills row 64*wave + 8*i + l/8, slot l%8,
    // i.e. global chunk (l%8) ^ swizzle(row); B likewise for bf16 rows; FP8:
    // row 64*wave + 16*i + l/4, slot l%4 (chunk (l%4) ^ swz8(row)); MXFP4:
    // row 64*wave + 32*i + l/2, slot l%2 (chunk (l%2) ^ ((row >> 3) & 1)),
    // and the exponent dword of row 64*wave + l
    // (second K segment: ao2, bo2; its A rows are the tile's rows)
    uint32_t ao[NDA], bo[NDB], ao2[KCAT ? NDA : 1], bo2[KCAT ? NDB : 1];
#pragma unroll
    for (int i = 0; i < NDA; ++i) {
        const int row = 64 * wave + 8 * i + (lane >> 3);
        const int chunk_bytes = swz(row, lane & 7) * 16;
        const int r = tc.row0 + row;
        const int rr = r < tc.row1 ? r : tc.row0;
        ao[i] = (uint32_t)(a_row_of(g, rr) * g.lda * 2) + chunk_bytes;
        if constexpr (KCAT) ao2[i] = (uint32_t)((int64_t)rr * g.lda2 * 2) + chunk_bytes;
    }
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        if constexpr (FP8) {
            const int row = 64 * wave + 16 * i + (lane >> 2);
            bo[i] = (uint32_t)((int64_t)wrow_of(row) * g.K) + swz8(row, lane & 3) * 16;
        } else if constexpr (FP4) {
            if (i < 2) {
                const int row = 64 * wave + 32 * i + (lane >> 1);
                bo[i] = (uint32_t)((int64_t)wrow_of(row) * (g.K / 2)) +
                        (((lane & 1) ^ ((row >> 3) & 1)) * 16);
            } else {
                bo[i] = (uint32_t)((int64_t)wrow_of(64 * wave + lane) * (g.K / 32));
            }
        } else {
            const int row = 64 * wave + 8 * i + (lane >> 3);
            bo[i] = (uint32_t)((int64_t)wrow_of(row) * g.K * 2) + swz(row, lane & 7) * 16;
            if constexpr (KCAT)
                bo2[i] = (uint32_t)((int64_t)wrow_of(row) * g.K2 * 2) + swz(row, lane & 7) * 16;
        }
    }
    const int nk1 = g.K / GBK;
    const int nk = nk1 + (KCAT ? g.K2 / GBK : 0);
    f32x16_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mi][nj][j] = 0.0f;

    // fragment (fr, fh): row fr, k 8*fh .. +7 of a 16-deep step, i.e. chunk
    // 2*ks + fh (FP8: half fh of chunk ks; MXFP4: bytes 8*ks + 4*fh .. +3
    // of the row); rows of the wave's blocks share their low 5 bits, so one
    // offset per step serves every block (the rest are immediates)
    const int fr = lane & 31, fh = lane >> 5;
    // Rows per compute wave: a tile of at most 128 (64) live rows gives each
    // wave 64 (32) of them, so that all four SIMDs share its MFMAs instead
    // of two (the DMA rows do not change)
    const int tile_rows = tc.row1 - tc.row0;
    const int wrows = tile_rows <= 64 ? 32 : tile_rows <= 128 ? 64 : 128;
    const int wrb = wrows * wm;  // the wave's first row in the tile
    const int arow0 = wrb + fr;
    const int brow0 = (SW ? 64 * wn : 128 * wn) + fr;
    int aoffs[4], boffs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int ch = 2 * ks + fh;
        aoffs[ks] = (arow0 * GBK + swz(arow0, ch) * 8) * 2;
        boffs[ks] = FP8   ? brow0 * GBK + swz8(brow0, ks) * 16 + fh * 8
                    : FP4 ? brow0 * 32 + (((ks >> 1) ^ ((brow0 >> 3) & 1)) * 16) + ((8 * ks + 4 * fh) & 15)
                          : (brow0 * GBK + swz(brow0, ch) * 8) * 2;
    }
    // row offset of B block nj from brow0: SwiGLU gate rows (nj 0, 1), then
    // the matching up rows
    auto bdrow = [](int nj) constexpr { return SW ? (nj < 2 ? 0 : 128) + 32 * (nj & 1) : 32 * nj; };
    // raw B fragment: bf16 values, 8 FP8 codes, or 8 E2M1 codes
    using braw_t = std::conditional_t<FP8, u32x2_t, std::conditional_t<FP4, uint32_t, bf16x8_t>>;
    struct Frags {
        bf16x8_t a[4];
        braw_t b[4];
    };
    const int nact = min(max((tile_rows - wrb + 31) / 32, 0), wrows / 32);

    auto run = [&](auto NAC) __attribute__((always_inline)) {
        constexpr int NA = decltype(NAC)::value;
        constexpr int NR = NA > 0 ? 4 + NA : 0;  // fragment reads per step
        // fragment read i of a step, in the order the step's MFMAs first use
        // them: A block 0, B blocks 0..3, then A blocks 1..NA-1
        auto rd1 = [&](int as, int bs, int ks, Frags& f, int i) __attribute__((always_inline)) {
            if (i >= 1 && i <= 4) {
                const int nj = i - 1;
                const char* b = smem + B_RING + bs + boffs[ks] + bdrow(nj) * B_ROW;
                f.b[nj] = *(const braw_t*)b;
            } else {
                const int mi = i == 0 ? 0 : i - 4;
                const char* a = smem + as + aoffs[ks];
                f.a[mi] = *(const bf16x8_t*)(a + mi * 32 * GBK * 2);
            }
        };
        // MXFP4: the exponent dword of each B block's row (four blocks, two
        // of which belong to the stage), read once per stage: stage 0's before
        // the loop, stage kt+1's during stage kt's last step
        uint32_t ex[4] = {0, 0, 0, 0};
        auto rde = [&](int bs, int nj) __attribute__((always_inline)) {
            ex[nj] = *(const uint32_t*)(smem + B_RING + bs + B_CODES + (brow0 + bdrow(nj)) * 4);
        };
        // bf16 B operands of a step, converted where first used
        bf16x8_t bc[4];
        auto conv = [&](const Frags& f, int kt, int ks, int nj) __attribute__((always_inline)) {
            if constexpr (FP8) {
                bc[nj] = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(f.b[nj][0], f.b[nj][1]));
            } else if constexpr (FP4) {
                // block 2kt + ks/2 is byte 2*(kt & 1) + ks/2 of the dword
                const uint32_t eb = (ex[nj] >> (8 * (2 * (kt & 1) + (ks >> 1)))) & 0xffu;
                bc[nj] = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16x8(f.b[nj], e8m0_scale(eb)));
            }
        };
        // MFMA i of a step: block (i / 4, i % 4); the first four MFMAs
        // convert the B fragment they introduce
        auto mf1 = [&](const Frags& f, int kt, int ks, int i) __attribute__((always_inline)) {
            if constexpr (FP8 || FP4) {
                if (i < 4) conv(f, kt, ks, i);
                acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    f.a[i >> 2], bc[i & 3], acc[i >> 2][i & 3], 0, 0, 0);
            } else {
                acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    f.a[i >> 2], f.b[i & 3], acc[i >> 2][i & 3], 0, 0, 0);
            }
        };
        // one DMA instruction of stage kt's A or B tile
        // (stage kt clamped to the last; the K segment picked with selects)
        auto da1 = [&](int as, int kt, int i) __attribute__((always_inline)) {
            char* dst = smem + as;
            kt = min(kt, nk - 1);
            const bool seg1 = !KCAT || kt < nk1;
            const char* abase = seg1 ? Ab : A2b;
            const uint32_t ko = (uint32_t)(seg1 ? kt : kt - nk1) * GBK * 2;
            __builtin_amdgcn_global_load_lds(
                (const void*)(abase + ((seg1 ? ao[i] : ao2[KCAT ? i : 0]) + ko)),
                (lds_ptr_t)(dst + (64 * wave + 8 * i) * GBK * 2), 16, 0, 0);
        };
        auto db1 = [&](int bs, int kt, int i) __attribute__((always_inline)) {
            char* dst = smem + B_RING + bs;
            kt = min(kt, nk - 1);
            if constexpr (FP8) {
                __builtin_amdgcn_global_load_lds((const void*)(Bb + (bo[i] + (uint32_t)kt * GBK)),
                                                 (lds_ptr_t)(dst + (64 * wave + 16 * i) * GBK), 16, 0, 0);
            } else if constexpr (FP4) {
                // the codes, then the exponent dword holding blocks 2kt, 2kt+1
                // (K is a multiple of 128, so that dword is aligned and whole)
                if (i < 2)
                    __builtin_amdgcn_global_load_lds((const void*)(Bb + (bo[i] + (uint32_t)kt * 32)),
                                                     (lds_ptr_t)(dst + (64 * wave + 32 * i) * 32), 16, 0, 0);
                else
                    __builtin_amdgcn_global_load_lds((const void*)(Sb + (bo[2] + (uint32_t)(kt >> 1) * 4)),
                                                     (lds_ptr_t)(dst + B_CODES + 64 * wave * 4), 4, 0, 0);
            } else {
                const bool seg1 = !KCAT || kt < nk1;
                const char* bbase = seg1 ? Bb : B2b;
                const uint32_t ko = (uint32_t)(seg1 ? kt : kt - nk1) * GBK * 2;
                __builtin_amdgcn_global_load_lds(
                    (const void*)(bbase + ((seg1 ? bo[i] : bo2[KCAT ? i : 0]) + ko)),
                    (lds_ptr_t)(dst + (64 * wave + 8 * i) * GBK * 2), 16, 0, 0);
            }
        };

        // DMA issue order: prologue A0 B0 A1 B1; turn kt issues B_{kt+2}
        // during its first step and A_{kt+2} during its last, after the
        // barrier that follows its third step.  Before the barrier of turn kt
        // (publishing stage kt+1) only B_{kt+2} may still be in flight.
#pragma unroll
        for (int i = 0; i < NDA; ++i) da1(0, 0, i);
#pragma unroll
        for (int i = 0; i < NDB; ++i) db1(0, 0, i);
#pragma unroll
        for (int i = 0; i < NDA; ++i) da1(A_BYTES, 1, i);
#pragma unroll
        for (int i = 0; i < NDB; ++i) db1(B_BYTES, 1, i);
        wait_vmcnt_lgkm0<NDA + NDB>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        Frags f0, f1;
        if constexpr (NA > 0) {
#pragma unroll
            for (int i = 0; i < NR; ++i) rd1(0, 0, 0, f0, i);
            if constexpr (FP4) {
#pragma unroll
                for (int nj = 0; nj < 4; ++nj) rde(0, nj);
            }
        }
        // ring slots (byte offsets) of stages kt, kt+1 (A) and kt, kt+1,
        // kt+2 (B), rotated at the end of each turn
        int sa0 = 0, sa1 = A_BYTES, sb0 = 0, sb1 = B_BYTES, sb2 = 2 * B_BYTES;
        for (int kt = 0; kt < nk; ++kt) {
            __builtin_amdgcn_sched_barrier(0);
            // step 0: MFMAs of f0, reads of step 1 and the B tile of kt+2,
            // one instruction after each MFMA
            {
                constexpr int NO = NR + NDB;
                constexpr int N0 = NA * 4 > NO ? NA * 4 : NO;
#pragma unroll
                for (int i = 0; i < N0; ++i) {
                    if (i < NA * 4) mf1(f0, kt, 0, i);
                    if (i < NR) rd1(sa0, sb0, 1, f1, i);
                    else if (i < NO) db1(sb2, kt + 2, i - NR);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (NA > 0) {
                // steps 1 and 2 (a one-block wave has 4 MFMAs for 5 reads)
                constexpr int N12 = NA * 4 > NR ? NA * 4 : NR;
#pragma unroll
                for (int i = 0; i < N12; ++i) {
                    if (i < NA * 4) mf1(f1, kt, 1, i);
                    if (i < NR) rd1(sa0, sb0, 2, f0, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < N12; ++i) {
                    if (i < NA * 4) mf1(f0, kt, 2, i);
                    if (i < NR) rd1(sa0, sb0, 3, f1, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            asm volatile("" ::: "memory");
            // stage kt+1 has landed for this wave and all its reads of stage
            // kt are retired; after the barrier stage kt+1 is visible and
            // stage kt's slots are free
            wait_vmcnt_lgkm0<NDB>();
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            // step 3 with the reads of stage kt+1's step 0 (and its
            // exponents) and the A tile of kt+2 (at the last turn the reads
            // take the clamped copy of the last stage: landed, never used)
            // (full waves: the A DMA after the even MFMAs, the reads after
            // the odd ones)
            {
                constexpr int M3 = NA * 4;
                // step 3's conversions use this stage's exponents: keep them
                // until its first four MFMAs have converted their fragments
                uint32_t exn[4] = {0, 0, 0, 0};
                auto rde3 = [&](int nj) __attribute__((always_inline)) {
                    exn[nj] = *(const uint32_t*)(smem + B_RING + sb1 + B_CODES + (brow0 + bdrow(nj)) * 4);
                };
                constexpr int NE = FP4 && NA > 0 ? 4 : 0;
                if constexpr (M3 >= 2 * (NR + NE) && M3 >= 2 * NDA) {
#pragma unroll
                    for (int i = 0; i < M3; ++i) {
                        mf1(f1, kt, 3, i);
                        if ((i & 1) == 0 && (i >> 1) < NDA) da1(sa0, kt + 2, i >> 1);
                        if ((i & 1) == 1 && (i >> 1) < NR) rd1(sa1, sb1, 0, f0, i >> 1);
                        else if ((i & 1) == 1 && (i >> 1) < NR + NE) rde3((i >> 1) - NR);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
                    constexpr int NO = NR + NE;
                    constexpr int N3 = M3 > NO ? (M3 > NDA ? M3 : NDA) : (NO > NDA ? NO : NDA);
#pragma unroll
                    for (int i = 0; i < N3; ++i) {
                        if (i < M3) mf1(f1, kt, 3, i);
                        if (i < NR) rd1(sa1, sb1, 0, f0, i);
                        else if (i < NO) rde3(i - NR);
                        if (i < NDA) da1(sa0, kt + 2, i);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if constexpr (FP4) {
#pragma unroll
                    for (int nj = 0; nj < 4; ++nj) ex[nj] = exn[nj];
                }
            }
            asm volatile("" ::: "memory");
            {
                const int t = sa0;
                sa0 = sa1;
                sa1 = t;
                const int u = sb0;
                sb0 = sb1;
                sb1 = sb2;
                sb2 = u;
            }
        }
        // the trailing DMAs must land before the LDS is reused
        wait_vmcnt<0>();
        __syncthreads();
        // FP8: the row scale of the weight row behind each block's column,
        // applied as the sums are written out
        float sn[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (FP8 && NA > 0) {
            const float* sc = (const float*)g.b_scale + (int64_t)tc.group * g.b_scale_gstride;
#pragma unroll
            for (int nj = 0; nj < 4; ++nj) sn[nj] = sc[wrow_of(brow0 + bdrow(nj))];
        }
        if constexpr (NA > 0) {
        // epilogue through LDS, one 32-row block at a time; row stride 136
        // floats (the two halves of a wave write 4 rows apart: banks +32)
        constexpr int ELD = 136;
        float* ep = (float*)smem + wave * 32 * ELD;
        constexpr int CW = EPI == EPI_F32 || EPI == EPI_F32_BIAS ? 4 : 8;
        constexpr int WC = SW ? 64 : 128;
        constexpr int LPR = WC / CW, RPI = 64 / LPR;
        const int c = (lane % LPR) * CW;
        const int col = SW ? tc.nt * 128 + 64 * wn + c : tc.nt * GBN + 128 * wn + c;
        const bool col_ok = col < g.N;
        auto epi = [&](auto ACTC) __attribute__((always_inline)) {
            constexpr int ACT = decltype(ACTC)::value;
#pragma unroll
            for (int mi = 0; mi < NA; ++mi) {
#pragma unroll
                for (int nj = 0; nj < 4; ++nj)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        ep[(8 * (j >> 2) + 4 * fh + (j & 3)) * ELD + nj * 32 + fr] =
                            FP8 ? acc[mi][nj][j] * sn[nj] : acc[mi][nj][j];
                asm volatile("" ::: "memory");
                const int rb = tc.row0 + wrb + mi * 32;
#pragma unroll
                for (int i = 0; i < 32 / RPI; ++i) {
                    const int row = i * RPI + lane / LPR;
                    const int r = rb + row;
                    const float* src = ep + row * ELD + c;
                    if (SW) {
                        const f32x4_t g0 = *(const f32x4_t*)(src);
                        const f32x4_t g1 = *(const f32x4_t*)(src + 4);
                        const f32x4_t u0 = *(const f32x4_t*)(src + 64);
                        const f32x4_t u1 = *(const f32x4_t*)(src + 68);
                        u32x4_t o;
                        o[0] = pack_bf16x2(glu_act<ACT>(g0[0], u0[0], g), glu_act<ACT>(g0[1], u0[1], g));
                        o[1] = pack_bf16x2(glu_act<ACT>(g0[2], u0[2], g), glu_act<ACT>(g0[3], u0[3], g));
                        o[2] = pack_bf16x2(glu_act<ACT>(g1[0], u1[0], g), glu_act<ACT>(g1[1], u1[1], g));
                        o[3] = pack_bf16x2(glu_act<ACT>(g1[2], u1[2], g), glu_act<ACT>(g1[3], u1[3], g));
                        if (r < tc.row1 && col_ok)
                            *(u32x4_t*)((bf16_t*)g.C + (int64_t)r * g.ldc + col) = o;
                    } else if (CW == 8) {
                        const f32x4_t v0 = *(const f32x4_t*)(src);
                        const f32x4_t v1 = *(const f32x4_t*)(src + 4);
                        u32x4_t o;
                        if (EPI == EPI_F16) {
                            o[0] = pack_f16x2(v0[0], v0[1]);
                            o[1] = pack_f16x2(v0[2], v0[3]);
                            o[2] = pack_f16x2(v1[0], v1[1]);
                            o[3] = pack_f16x2(v1[2], v1[3]);
                        } else {
                            o[0] = pack_bf16x2(v0[0], v0[1]);
                            o[1] = pack_bf16x2(v0[2], v0[3]);
                            o[2] = pack_bf16x2(v1[0], v1[1]);
                            o[3] = pack_bf16x2(v1[2], v1[3]);
                        }
                        if (r < tc.row1 && col_ok)
                            *(u32x4_t*)((uint16_t*)g.C + (int64_t)r * g.ldc + col) = o;
                    } else {
                        f32x4_t v = *(const f32x4_t*)(src);
                        if (EPI == EPI_F32_BIAS && g.bias && col_ok) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] += g.bias[col + t];
                        }
                        if (r < tc.row1 && col_ok)
                            *(f32x4_t*)((float*)g.C + (int64_t)r * g.ldc + col) = v;
                    }
                }
                asm volatile("" ::: "memory");
            }
        };
        if constexpr (SW) with_act(g, epi);
        else epi(std::integral_constant<int, ACT_SILU>{});
        }
    };
    if (nact == 4) run(std::integral_constant<int, 4>{});
    else if (nact == 3) run(std::integral_constant<int, 3>{});
    else if (nact == 2) run(std::integral_constant<int, 2>{});
    else if (nact == 1) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
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
    for (int j = 0; j < 4; ++j)
        bcol[j] = SW ? (j < 2 ? tx * 2 + j : 32 + tx * 2 + j - 2) : tx * 4 + j;

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
                    ((float*)g.C)[(int64_t)r * g.ldc + hc] = glu_f32<true>(gt, up, g);
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
    const dim3 bd(256);
    if constexpr (KC) {
        // the K-concatenated dense product (no fp16 rows)
        switch (g.epi) {
            case EPI_F32: gemm_bf16_big4<EPI_F32, WF_BF16, true><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32_BIAS: gemm_bf16_big4<EPI_F32_BIAS, WF_BF16, true><<<gd, bd, 0, s>>>(g); break;
            case EPI_OUT: gemm_bf16_big4<EPI_OUT, WF_BF16, true><<<gd, bd, 0, s>>>(g); break;
            default: gemm_bf16_big4<EPI_SWIGLU, WF_BF16, true><<<gd, bd, 0, s>>>(g); break;
        }
    } else if (g.b_fmt == WF_FP8) {
        // grouped expert products only: gate/up, and the down product's rows
        switch (g.epi) {
            case EPI_F16: gemm_bf16_big4<EPI_F16, WF_FP8, false><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32: gemm_bf16_big4<EPI_F32, WF_FP8, false><<<gd, bd, 0, s>>>(g); break;
            default: gemm_bf16_big4<EPI_SWIGLU, WF_FP8, false><<<gd, bd, 0, s>>>(g); break;
        }
    } else if (g.b_fmt == WF_MXFP4) {
        switch (g.epi) {
            case EPI_F16: gemm_bf16_big4<EPI_F16, WF_MXFP4, false><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32: gemm_bf16_big4<EPI_F32, WF_MXFP4, false><<<gd, bd, 0, s>>>(g); break;
            default: gemm_bf16_big4<EPI_SWIGLU, WF_MXFP4, false><<<gd, bd, 0, s>>>(g); break;
        }
    } else {
        switch (g.epi) {
            case EPI_F16: gemm_bf16_big4<EPI_F16, WF_BF16, false><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32: gemm_bf16_big4<EPI_F32, WF_BF16, false><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32_BIAS: gemm_bf16_big4<EPI_F32_BIAS, WF_BF16, false><<<gd, bd, 0, s>>>(g); break;
            case EPI_OUT: gemm_bf16_big4<EPI_OUT, WF_BF16, false><<<gd, bd, 0, s>>>(g); break;
            default: gemm_bf16_big4<EPI_SWIGLU, WF_BF16, false><<<gd, bd, 0, s>>>(g); break;
        }
    }
}

}  // namespace

hipError_t launch_tiled_kslices(const GemmArgs& g, int kslices, hipStream_t s) {
    if (g.tiles || g.A2 || g.b_fmt != WF_BF16 || g.epi != EPI_F32 || kslices < 1 ||
        kslices > g.K / TBK)
        return hipErrorInvalidValue;
    const int nm = (g.M + TBM - 1) / TBM;
    const dim3 gd((unsigned)((int64_t)nm * ((g.N + TBN - 1) / TBN)), (unsigned)kslices), bd(256);
    if (nm > 0) gemm_bf16_tiled<EPI_F32><<<gd, bd, 0, s>>>(g);
    return hipGetLastError();
}

namespace {

int col_tiles(int path, int dtype, int epi, int N) {
    const bool sw = epi == EPI_SWIGLU;
    if (dtype == 0) return sw ? (N + 31) / 32 : (N + FBN - 1) / FBN;
    if (path == GEMM_STREAM) return stream_col_tiles(epi, N);
    if (path == GEMM_BIG) return sw ? (N + 127) / 128 : (N + GBN - 1) / GBN;
    return sw ? (N + 63) / 64 : (N + TBN - 1) / TBN;
}

int row_tile(int path, int dtype) {
    if (dtype == 0) return FBM;
    if (path == GEMM_STREAM) return stream_row_tile();
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
    if (g.b_fmt != WF_BF16 && (dtype == 0 || g.A2)) return hipErrorInvalidValue;
    // the 256x256 kernel takes quantised weights for grouped gate/up or
    // expert rows only
    if (path == GEMM_BIG && g.b_fmt != WF_BF16 &&
        (!g.tiles || (g.epi != EPI_SWIGLU && g.epi != EPI_F16 && g.epi != EPI_F32)))
        return hipErrorInvalidValue;
    // fp16 expert rows: grouped bf16 products without a second K segment
    if (g.epi == EPI_F16 && (dtype == 0 || !g.tiles || g.A2)) return hipErrorInvalidValue;
    // the 128x128 kernel takes bf16 weights and stores no fp16 expert rows
    if (dtype != 0 && path == GEMM_TILED && (g.b_fmt != WF_BF16 || g.epi == EPI_F16))
        return hipErrorInvalidValue;
    if (g.b_fmt == WF_MXFP4 && g.K % 128 != 0) return hipErrorInvalidValue;
    if (dtype == 0) {
        MOE_GEMM_SWITCH(gemm_f32_tiled)
    } else if (path == GEMM_STREAM) {
        return launch_stream_gemm(g, nm, s);
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
