// Grouped GEMM for expert groups of more than 64 rows, on gfx950: 256x256
// tiles whose weight operand streams from global memory straight into
// registers, while the token operand goes through a 4-deep LDS ring.
//
// The product is a grouped matmul of the expert MLP ("vLLM-Ascend Kimi K3 MoE
// Forward Insight", Stage 4: gate/up matmul -> activation -> down matmul):
//     C[r, n] = sum_k A[arow(r), k] * B_g[n, k],
// A the gathered token rows (x, or h for the down product), B_g the group's
// weights [N, K] (K-contiguous), the epilogue fused (SwiGLU or another gate/up
// activation into h; fp16 or fp32 expert rows for the down product).
//
// Layout.  One workgroup of 4 waves (one per SIMD) takes 256 token rows and
// 256 weight rows; wave w owns weight rows 64w .. 64w+63 of the tile against
// all 256 token rows (for SwiGLU: 32 gate rows and the 32 up rows of the same
// h columns, so the activation is formed in registers).  The products are
// v_mfma_f32_16x16x32_bf16 with the weights as the 16-row first operand and
// 16 tokens as the second: 16 token blocks x 4 weight blocks = 64 fp32
// accumulator tiles (256 registers) per wave.
//
// Why this shape.  A 256x256 tile with both operands in LDS reads 192 KB of
// LDS fragments per 64-deep K stage and, with 64 KB per stage, leaves room
// for only two ring slots: each stage's DMA has one stage of MFMA time to
// land before the barrier that publishes it.  Here the weights, which are
// not shared between the waves, go from global memory to registers in the
// MFMA operand layout (16 rows x 64 bytes per instruction, the pattern that
// streams HBM at its full rate), four stages ahead of their use.  Only the
// token operand (32 KB per stage) lives in LDS, so the ring has four slots
// and each stage's token DMA has three stages to land; each wave reads 32 KB
// of token fragments per stage (128 KB for the CU, against 192 KB).
//
// Token stages are filled by global_load_lds in whole 128-byte lines (8 rows
// x 128 bytes per instruction).  LDS row r keeps its eight 16-byte chunks at
// chunk ^ ((r & 7) ^ ((r >> 3) & 1)); a fragment read (16 rows, one chunk)
// then hits 16 distinct 16-byte bank groups, free of conflicts with 32 or 64
// banks.  Token rows past the tile's end load the tile's first row (never
// stored), and token blocks wholly past it are skipped.
#include "gemm_tiles.h"

namespace moe {

namespace {

using namespace tiles;

constexpr int RBM = 256;                  // token rows per tile
constexpr int RBN = 256;                  // weight rows per tile
constexpr int RBK = 64;                   // k per stage
constexpr int RSLOTS = 4;                 // token ring slots = weight register stages
constexpr int RSTAGE = RBM * RBK * 2;     // bytes of one token stage (32 KB)

__device__ __forceinline__ int rw_swz(int row, int chunk) {
    return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_rw(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + 127) / 128 : (g.N + RBN - 1) / RBN;
    TileCoord tc;
    if (!fetch_tile(g, RBM, ntn, tc)) return;

    __shared__ __attribute__((aligned(1024))) char smem[RSLOTS * RSTAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    // token blocks of 16 rows that hold rows of the tile (1..16)
    const int ntb = (tc.row1 - tc.row0 + 15) >> 4;

    // Token DMA: wave w fills tile rows 64w .. 64w+63 of each stage with 8
    // instructions of 8 rows; lane l writes row +l/8, LDS chunk l%8, i.e. it
    // fetches the global chunk whose swizzled slot that is.  32-bit byte
    // offsets from a uniform base (every operand is under 4 GiB).
    const char* Ab = (const char*)g.A;
    uint32_t ao[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + (lane >> 3);
        const int r = tc.row0 + row;
        const int rr = r < tc.row1 ? r : tc.row0;
        ao[i] = (uint32_t)(a_row_of(g, rr) * g.lda * 2) + rw_swz(row, lane & 7) * 16;
    }

    // Weight rows of this wave: 4 blocks of 16.  SwiGLU: blocks 0-1 are gate
    // rows of h columns hc0 .. hc0+31, blocks 2-3 the up rows of the same
    // columns.  Rows past N read row N-1 (never stored).  Lane l reads row
    // l%16 of a block, 16 bytes at k-chunk l/16 of each 32-deep step.
    const char* Bb = (const char*)g.B + (int64_t)tc.group * g.b_gstride * 2;
    uint32_t bo[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        int wrow;
        if (SW) {
            const int c = min(tc.nt * 128 + wave * 32 + (f & 1) * 16 + l16, g.N - 1);
            wrow = f < 2 ? c : g.N + c;
        } else {
            wrow = min(tc.nt * RBN + wave * 64 + f * 16 + l16, g.N - 1);
        }
        bo[f] = (uint32_t)((int64_t)wrow * g.K * 2) + g4 * 16;
    }

    const int nk = g.K / RBK;

    // stage kt's token DMA into slot kt % 4 (stages past the end re-read the
    // last one, so that every stage issues the same number of loads)
    auto issue_a = [&](int kt) __attribute__((always_inline)) {
        const int slot = kt & (RSLOTS - 1);
        const uint32_t ko = (uint32_t)min(kt, nk - 1) * (RBK * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void*)(Ab + (ao[i] + ko)),
                (lds_ptr_t)(smem + slot * RSTAGE + (64 * wave + 8 * i) * 128), 16, 0, 0);
    };
    // stage kt's weight fragments: [block f][step s]
    u32x4_t bw[RSLOTS][4][2];
    auto load_b = [&](int kt, u32x4_t (&dst)[4][2]) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)min(kt, nk - 1) * (RBK * 2);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                dst[f][s] = *(const u32x4_t*)(Bb + (bo[f] + ko + s * 64));
    };

    f32x4_t acc[16][4];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[j][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // LDS byte offset of this lane's token fragment (block j, step s) inside
    // a stage: row 16j + l16, chunk 4s + g4.  The swizzle reads bits 0..3 of
    // the row only, so block j sits at a constant 2 KB step from block 0.
    uint32_t xoff[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) xoff[s] = (uint32_t)(l16 * 128 + rw_swz(l16, 4 * s + g4) * 16);

    // One stage against the first NJ token blocks (the blocks past the
    // tile's last row are skipped in steps of 4: NJ = 4, 8, 12 or 16).
    auto compute = [&](auto NJc, int slot, const u32x4_t (&b)[4][2])
                       __attribute__((always_inline)) {
        constexpr int NJ = decltype(NJc)::value;
        const char* xs = smem + slot * RSTAGE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8_t wf[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) wf[f] = __builtin_bit_cast(bf16x8_t, b[f][s]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bf16x8_t xv = *(const bf16x8_t*)(xs + xoff[s] + j * 2048);
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    acc[j][f] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[f], xv, acc[j][f], 0, 0, 0);
            }
        }
    };

    // Stages 0..2 go out before the loop; stage kt + 3 after the barrier of
    // stage kt, into the slot (and weight registers) stage kt - 1 used.  Per
    // stage each wave issues 8 token DMA and 8 weight loads, so when stage kt
    // starts exactly the 32 loads of stages kt+1 and kt+2 may still be in
    // flight.  The loop body covers four stages, so that ring slots and
    // weight registers are static; the last nk % 4 stages follow it.
    auto stage = [&](auto NJc, int kt, auto Uc) __attribute__((always_inline)) {
        constexpr int u = decltype(Uc)::value;
        // this wave's token DMA and weights of stage kt have landed, and its
        // LDS reads of stage kt-1 are done; after the barrier every wave's
        // part of stage kt is visible and slot (kt-1)%4 is free
        wait_vmcnt_lgkm0<32>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_a(kt + 3);
        load_b(kt + 3, bw[(u + 3) & (RSLOTS - 1)]);
        asm volatile("" ::: "memory");
        compute(NJc, u, bw[u]);
    };
    auto run = [&](auto NJc) __attribute__((always_inline)) {
        issue_a(0);
        load_b(0, bw[0]);
        issue_a(1);
        load_b(1, bw[1]);
        issue_a(2);
        load_b(2, bw[2]);
        using U0 = std::integral_constant<int, 0>;
        using U1 = std::integral_constant<int, 1>;
        using U2 = std::integral_constant<int, 2>;
        using U3 = std::integral_constant<int, 3>;
        int kt = 0;
        for (; kt + RSLOTS <= nk; kt += RSLOTS) {
            stage(NJc, kt, U0{});
            stage(NJc, kt + 1, U1{});
            stage(NJc, kt + 2, U2{});
            stage(NJc, kt + 3, U3{});
        }
        const int rem = nk - kt;
        if (rem > 0) stage(NJc, kt, U0{});
        if (rem > 1) stage(NJc, kt + 1, U1{});
        if (rem > 2) stage(NJc, kt + 2, U2{});
    };
    if (ntb > 12) run(std::integral_constant<int, 16>{});
    else if (ntb > 8) run(std::integral_constant<int, 12>{});
    else if (ntb > 4) run(std::integral_constant<int, 8>{});
    else run(std::integral_constant<int, 4>{});

    // the trailing token DMA must land before the workgroup's LDS goes away
    wait_vmcnt<0>();

    // Epilogue straight from the accumulators: acc[j][f][i] = C[token 16j +
    // l16][weight row 16f + 4*g4 + i of this wave], four consecutive output
    // columns per lane (8 or 16 bytes).
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = tc.row0 + 16 * j + l16;
        if (j >= ntb || r >= tc.row1) continue;
        if (SW) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const int hc = tc.nt * 128 + wave * 32 + f * 16 + 4 * g4;
                if (hc >= g.N) continue;
                const f32x4_t gt = acc[j][f], up = acc[j][f + 2];
                uint2 o;
                o.x = pack_bf16x2(glu_f32(gt[0], up[0], g), glu_f32(gt[1], up[1], g));
                o.y = pack_bf16x2(glu_f32(gt[2], up[2], g), glu_f32(gt[3], up[3], g));
                *(uint2*)((bf16_t*)g.C + (int64_t)r * g.ldc + hc) = o;
            }
        } else {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int c = tc.nt * RBN + wave * 64 + f * 16 + 4 * g4;
                if (c >= g.N) continue;
                f32x4_t v = acc[j][f];
                if (EPI == EPI_F32_BIAS && g.bias) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] += g.bias[c + i];
                }
                if (EPI == EPI_OUT) {
                    *(uint2*)((bf16_t*)g.C + (int64_t)r * g.ldc + c) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                } else if (EPI == EPI_F16) {
                    *(uint2*)((uint16_t*)g.C + (int64_t)r * g.ldc + c) =
                        make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
                } else {
                    *(f32x4_t*)((float*)g.C + (int64_t)r * g.ldc + c) = v;
                }
            }
        }
    }
}

}  // namespace

int rw_row_tile() { return RBM; }

hipError_t launch_rw_gemm(const GemmArgs& g, int nm, hipStream_t s) {
    // bf16 weights, one K segment, widths multiples of 64 (checked by the
    // entry points); the tile list (if any) was built with 256-row tiles
    if (g.b_fmt != WF_BF16 || g.A2 || g.K % RBK != 0 || g.N % 4 != 0)
        return hipErrorInvalidValue;
    const int ntn = g.epi == EPI_SWIGLU ? (g.N + 127) / 128 : (g.N + RBN - 1) / RBN;
    const int64_t grid = (int64_t)nm * ntn;
    if (grid <= 0) return hipSuccess;
    const dim3 gd((unsigned)grid), bd(256);
    switch (g.epi) {
        case EPI_F32: gemm_bf16_rw<EPI_F32><<<gd, bd, 0, s>>>(g); break;
        case EPI_F32_BIAS: gemm_bf16_rw<EPI_F32_BIAS><<<gd, bd, 0, s>>>(g); break;
        case EPI_OUT: gemm_bf16_rw<EPI_OUT><<<gd, bd, 0, s>>>(g); break;
        case EPI_F16: gemm_bf16_rw<EPI_F16><<<gd, bd, 0, s>>>(g); break;
        default: gemm_bf16_rw<EPI_SWIGLU><<<gd, bd, 0, s>>>(g); break;
    }
    return hipGetLastError();
}

}  // namespace moe
