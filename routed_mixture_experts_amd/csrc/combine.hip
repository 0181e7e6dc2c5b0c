// Combine: back to token order with the routing weights applied
// ("vLLM-Ascend Kimi K3 MoE Forward Insight", Stage 4 mode table, AllGather
// row: combine restores token order and applies the probabilities).
//
//   out[t, d] = sum_{j = 0..k-1} w[t, j] * y_rows[pair_to_row[t*k + j], d]
//
// A gather, not a scatter: every output element is owned by one thread, the
// k rows are read through the inverse permutation, the sum runs in fp32 in
// ascending j and is rounded once.  No atomics.  The expert rows come in
// fp32 or fp16 (bf16 layers; every fp16 value is exact in fp32).  Optional
// fused extras:
//  * an fp32 addend (the shared expert's output) added before the rounding;
//  * RMSNorm of the whole row (the latent tail's norm, page
//    "vllm.models.kimi_k3.nvidia.latent_moe_runner", allreduce_norm_latent_out
//    at tensor-parallel size 1), y * rsqrt(mean(y^2) + eps) * gamma in fp32,
//    in which case one workgroup keeps the whole row in registers.
#include "common.h"

namespace moe {

namespace {

__device__ __forceinline__ void store4(void* out, int out_dtype, int64_t idx, f32x4_t v) {
    if (out_dtype == 0) {
        *(f32x4_t*)((float*)out + idx) = v;
    } else {
        uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        *(uint2*)((bf16_t*)out + idx) = make_uint2(lo, hi);
    }
}

// Four consecutive values of expert row `row` from fp32 or fp16 storage.
__device__ __forceinline__ f32x4_t load_y4(const CombineArgs& a, int64_t row, int d) {
    if (a.y_f16) {
        const uint2 h = *(const uint2*)((const uint16_t*)a.y_rows + row * a.D + d);
        return f32x4_t{f16_bits_to_f32(h.x & 0xffffu), f16_bits_to_f32(h.x >> 16),
                       f16_bits_to_f32(h.y & 0xffffu), f16_bits_to_f32(h.y >> 16)};
    }
    return *(const f32x4_t*)((const float*)a.y_rows + row * a.D + d);
}

__device__ __forceinline__ float gamma_at(const void* gamma, int out_dtype, int d) {
    return out_dtype == 0 ? ((const float*)gamma)[d] : bf16_to_f32(((const bf16_t*)gamma)[d]);
}

// grid (T, ceil(D / 1024)); each thread one float4 of one token row.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    __shared__ int rows[kMaxTopK];
    __shared__ float ws[kMaxTopK];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < a.k) {
        rows[tid] = a.pair_to_row[t * a.k + tid];
        ws[tid] = a.weights[t * a.k + tid];
    }
    __syncthreads();
    const int d = (blockIdx.y * 256 + tid) * 4;
    if (d >= a.D) return;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; ++j) {
        const f32x4_t v = load_y4(a, rows[j], d);
        const float w = ws[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, v[i], acc[i]);
    }
    if (a.addend) {
        const f32x4_t s = *(const f32x4_t*)(a.addend + t * a.D + d);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += s[i];
    }
    store4(a.out, a.out_dtype, t * a.D + d, acc);
}

// fp16 expert rows, D a multiple of 8, 16-byte aligned operands: each
// thread eight values of one token row, so every row piece is one 16-byte
// load (a wave reads 1 KB of a row) and a bf16 output one 16-byte store;
// same sums, same order.  Grid (T, ceil(D / 1024)), 128 threads.
__global__ __launch_bounds__(128) void combine_f16x8_kernel(CombineArgs a) {
    __shared__ int rows[kMaxTopK];
    __shared__ float ws[kMaxTopK];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < a.k) {
        rows[tid] = a.pair_to_row[t * a.k + tid];
        ws[tid] = a.weights[t * a.k + tid];
    }
    __syncthreads();
    const int d = (blockIdx.y * 128 + tid) * 8;
    if (d >= a.D) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; ++j) {
        const uint4 h = *(const uint4*)((const uint16_t*)a.y_rows + (int64_t)rows[j] * a.D + d);
        const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
        const float w = ws[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w, f16_bits_to_f32(hw[i] & 0xffffu), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, f16_bits_to_f32(hw[i] >> 16), acc[2 * i + 1]);
        }
    }
    if (a.addend) {
        const f32x4_t s0 = *(const f32x4_t*)(a.addend + t * a.D + d);
        const f32x4_t s1 = *(const f32x4_t*)(a.addend + t * a.D + d + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += s0[i], acc[4 + i] += s1[i];
    }
    if (a.out_dtype == 0) {
        *(f32x4_t*)((float*)a.out + t * a.D + d) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *(f32x4_t*)((float*)a.out + t * a.D + d + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    } else {
        *(uint4*)((bf16_t*)a.out + t * a.D + d) =
            make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

// One workgroup per token; the row (D <= 1024 * NV) stays in registers.
template <int NV>
__global__ __launch_bounds__(256) void combine_norm_kernel(CombineArgs a) {
    __shared__ int rows[kMaxTopK];
    __shared__ float ws[kMaxTopK];
    __shared__ float part[4];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < a.k) {
        rows[tid] = a.pair_to_row[t * a.k + tid];
        ws[tid] = a.weights[t * a.k + tid];
    }
    __syncthreads();
    f32x4_t acc[NV];
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int d = (v * 256 + tid) * 4;
        if (d < a.D) {
            for (int j = 0; j < a.k; ++j) {
                const f32x4_t y = load_y4(a, rows[j], d);
                const float w = ws[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[v][i] = fmaf(w, y[i], acc[v][i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = fmaf(acc[v][i], acc[v][i], ss);
        }
    }
    // block sum of squares: wave tree, then 4 partials in a fixed order
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = 1.0f / sqrtf(tot / (float)a.D + a.eps);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int d = (v * 256 + tid) * 4;
        if (d >= a.D) continue;
        f32x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc[v][i] * inv * gamma_at(a.gamma, a.out_dtype, d + i);
        store4(a.out, a.out_dtype, t * a.D + d, o);
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    if (a.gamma) {
        const int nv = (a.D + 1023) / 1024;
        dim3 grid((unsigned)a.T), block(256);
        if (nv <= 1) combine_norm_kernel<1><<<grid, block, 0, s>>>(a);
        else if (nv <= 2) combine_norm_kernel<2><<<grid, block, 0, s>>>(a);
        else if (nv <= 4) combine_norm_kernel<4><<<grid, block, 0, s>>>(a);
        else combine_norm_kernel<8><<<grid, block, 0, s>>>(a);
    } else if (a.y_f16 && a.D % 8 == 0 &&
               (((uintptr_t)a.y_rows | (uintptr_t)a.out | (uintptr_t)a.addend) & 15) == 0) {
        dim3 grid((unsigned)a.T, (unsigned)((a.D + 1023) / 1024)), block(128);
        combine_f16x8_kernel<<<grid, block, 0, s>>>(a);
    } else {
        dim3 grid((unsigned)a.T, (unsigned)((a.D + 1023) / 1024)), block(256);
        combine_kernel<<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace moe
