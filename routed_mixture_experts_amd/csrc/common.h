// Internal declarations shared by the HIP translation units of the routed-MoE
// library (gfx950 only).  Nothing here is part of the C ABI.
#pragma once

#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;   // IEEE bfloat16 bit pattern

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxGroups = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

// Round to nearest even (inputs are finite in this library).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// IEEE binary16 bit patterns: fp32 -> fp16 rounds to nearest even
// (v_cvt_f16_f32); fp16 -> fp32 is exact.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Tile-list entry of a grouped GEMM: rows [row0, row1) of group g; the
// group's tiles are the contiguous entries [first, first + count).
struct Tile {
    int32_t group, row0, row1, first, count, pad0, pad1, pad2;
};

// Epilogues of the GEMM kernels.
enum Epilogue : int {
    EPI_F32 = 0,        // C f32 [M, N]
    EPI_F32_BIAS = 1,   // C f32 [M, N] = acc + bias[n]
    EPI_OUT = 2,        // C in the layer dtype [M, N]
    EPI_SWIGLU = 3,     // C in the layer dtype [M, N]: silu(acc_gate) * acc_up
    EPI_F16 = 4         // C fp16 [M, N] (the expert rows of bf16 layers; grouped only)
};

// One GEMM launch: C[r, n] = sum_k A[arow(r), k] * B_g[n, k]
//   (+ sum_k A2[r, k] * B2[n, k] when a second K segment is given).
// A rows: a_map ? a_map[r] / a_div : r.  B_g = B + g * b_gstride elements,
// row-major [Nb, K].  For EPI_SWIGLU, B_g holds 2N rows (gate rows, then up
// rows) and C has N columns.
struct GemmArgs {
    const void* A;
    int64_t lda;
    const int32_t* a_map;
    int32_t a_div;
    const void* B;
    int64_t b_gstride;
    int32_t K;
    const void* A2;   // optional second K segment (dense rows only)
    int64_t lda2;
    const void* B2;
    int32_t K2;
    int32_t N;
    int32_t M;                 // dense row count (ignored when tiles != null)
    const Tile* tiles;         // grouped tile list (null: dense)
    const int32_t* num_tiles;  // device count of valid tiles
    int32_t max_tiles;         // upper bound used for the grid
    int32_t tile_m;            // rows per tile the list was built with
    int32_t epi;
    void* C;
    int64_t ldc;
    const float* bias;
    // Storage of B (WeightFmt).  WF_FP8: OCP e4m3 codes, one byte per
    // element, and one fp32 scale per B row: row n of group g is scaled by
    // ((const float*)b_scale)[g * b_scale_gstride + n].  WF_MXFP4: OCP E2M1
    // codes, two per byte (element 2j in the low nibble of byte j of the row),
    // and one E8M0 byte per 32 elements of a row: block b of row n of group g
    // is scaled by 2^(e - 127), e = ((const uint8_t*)b_scale)[g *
    // b_scale_gstride + n * (K / 32) + b].  b_gstride counts elements.
    int32_t b_fmt;
    const void* b_scale;
    int64_t b_scale_gstride;
    // gate/up activation of EPI_SWIGLU (GluAct) and its parameters
    int32_t act;
    float act_alpha, act_limit;
};

enum WeightFmt { WF_BF16 = 0, WF_FP8 = 1, WF_MXFP4 = 2 };

// Gate/up activations h = act(gate, up) ("vLLM-Ascend Kimi K3 MoE Forward
// Insight", Stage 4: the MLP's activation branches): SwiGLU silu(g) * u;
// GELU (erf form) and its tanh approximation, gelu(g) * u; and the clipped
// SwiGLU min(g, L) * sigmoid(alpha * min(g, L)) * (clamp(u, -L, L) + 1).
enum GluAct { ACT_SILU = 0, ACT_GELU = 1, ACT_GELU_TANH = 2, ACT_SWIGLU_CLIP = 3 };

// One activation, fixed at compile time.  PRECISE: exact division for the
// fp32 layer; otherwise the hardware reciprocal.
template <int ACT, bool PRECISE = false>
__device__ __forceinline__ float glu_act(float gt, float up, const GemmArgs& a) {
    auto sigmoid = [](float v) {
        return PRECISE ? 1.0f / (1.0f + expf(-v)) : __builtin_amdgcn_rcpf(1.0f + __expf(-v));
    };
    if constexpr (ACT == ACT_GELU) {
        return 0.5f * gt * (1.0f + erff(gt * 0.70710678118654752f)) * up;
    } else if constexpr (ACT == ACT_GELU_TANH) {
        const float z = 0.79788456080286536f * (gt + 0.044715f * gt * gt * gt);
        return 0.5f * gt * (1.0f + tanhf(z)) * up;
    } else if constexpr (ACT == ACT_SWIGLU_CLIP) {
        const float gc = fminf(gt, a.act_limit);
        const float uc = fminf(fmaxf(up, -a.act_limit), a.act_limit);
        return gc * sigmoid(a.act_alpha * gc) * (uc + 1.0f);
    } else {
        return PRECISE ? gt / (1.0f + expf(-gt)) * up : gt * sigmoid(gt) * up;
    }
}

// The activation picked per element from the launch's code (uniform over the
// launch: one scalar branch per element).  Epilogues with many elements per
// lane switch once outside their loops and call glu_act instead.
template <bool PRECISE = false>
__device__ __forceinline__ float glu_f32(float gt, float up, const GemmArgs& a) {
    switch (a.act) {
        case ACT_GELU: return glu_act<ACT_GELU, PRECISE>(gt, up, a);
        case ACT_GELU_TANH: return glu_act<ACT_GELU_TANH, PRECISE>(gt, up, a);
        case ACT_SWIGLU_CLIP: return glu_act<ACT_SWIGLU_CLIP, PRECISE>(gt, up, a);
        default: return glu_act<ACT_SILU, PRECISE>(gt, up, a);
    }
}

// Calls body(std::integral_constant<int, ACT>{}) for the launch's activation.
template <typename F>
__device__ __forceinline__ void with_act(const GemmArgs& a, F&& body) {
    switch (a.act) {
        case ACT_GELU: body(std::integral_constant<int, ACT_GELU>{}); break;
        case ACT_GELU_TANH: body(std::integral_constant<int, ACT_GELU_TANH>{}); break;
        case ACT_SWIGLU_CLIP: body(std::integral_constant<int, ACT_SWIGLU_CLIP>{}); break;
        default: body(std::integral_constant<int, ACT_SILU>{}); break;
    }
}

// ----- launchers (return hipSuccess or the launch error) -----
struct RouteArgs {
    int64_t T;
    int32_t E, k, G, topk_group, score, group_score, renormalize;
    float scaling;
    int32_t raw_keys;
    const float* logits;
    const float* bias;
    int32_t* ids;
    float* weights;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

int permute_chunks(int64_t P);
hipError_t launch_permute(int64_t P, int32_t E, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* row_to_pair, int32_t* pair_to_row,
                          int32_t* chunk_scratch, hipStream_t s);
// Splits the groups into a small-tile list (one tile per group of 1..small_max
// rows) and a big-tile list (big_m-row tiles of the larger groups).
// phys[p] = log2phy[ids[p]] (both clamped into range).
hipError_t launch_log2phy(int64_t P, const int32_t* ids, const int32_t* log2phy,
                          int32_t num_logical, int32_t num_physical, int32_t* phys,
                          hipStream_t s);
// load[e] += counts[e] for e < n.
hipError_t launch_load_accumulate(int32_t n, const int32_t* counts, int64_t* load, hipStream_t s);
hipError_t launch_build_tiles(const int32_t* offsets, int32_t E, int32_t small_max,
                              int32_t big_m, Tile* small_tiles, int32_t* num_small,
                              Tile* big_tiles, int32_t* num_big, hipStream_t s);

// dtype: 0 = f32, 1 = bf16.  path: see gemm.hip (chosen by the caller).
enum GemmPath : int { GEMM_TILED = 0, GEMM_STREAM = 1, GEMM_BIG = 2 };
hipError_t launch_gemm(int dtype, int path, const GemmArgs& g, hipStream_t s);
// The weight-streaming kernels (gemm_stream.hip): rows per tile, column tiles,
// and the launch over nm row tiles.
int stream_row_tile();
int stream_col_tiles(int epi, int N);
hipError_t launch_stream_gemm(const GemmArgs& g, int nm, hipStream_t s);
// Rows per tile of a kernel (a grouped tile list must be built with it).
int gemm_row_tile(int dtype, int path);
// Largest group the streaming kernel takes as a single tile.
constexpr int kStreamMaxRows = 64;

struct CombineArgs {
    int64_t T;
    int32_t k, D;
    const void* y_rows;      // [T*k, D] f32, or fp16 when y_f16
    int32_t y_f16;
    const int32_t* pair_to_row;
    const float* weights;
    const float* addend;     // optional [T, D] f32 added before rounding
    const void* gamma;       // optional: fused RMSNorm (layer dtype)
    float eps;
    int32_t out_dtype;       // 0 f32, 1 bf16
    void* out;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace moe
