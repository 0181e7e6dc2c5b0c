// Router logits l = x W_r^T (+ bias row) of a small batch ("vLLM-Ascend Kimi
// K3 MoE Forward Insight", Mermaid flowchart: the gate produces router_logits
// before expert selection; bf16 inputs, fp32 sums and output).
//
// With few tokens the product is a stream of W_r (E x H) against a handful of
// token rows.  Whole-row or 4-way K-split streams give only E/64 x T/16
// workgroups (48 for 384 experts and 128 tokens), too few to keep loads in
// flight on 256 CUs.  Here a workgroup takes 16 experts (one MFMA block) and
// one K slice of up to 16 k-steps; each of its 4 waves loads its 4 steps (2
// above 128 tokens) at once, so it waits for one memory latency, applies
// each weight fragment to all token blocks (v_mfma_f32_16x16x32_bf16,
// weights as the first operand), and the waves' sums meet in LDS.  Each slice writes its partial sums; a second
// kernel adds the slices in order, so the result does not depend on
// scheduling.
#include "router.h"

#include <string.h>

#include <algorithm>

namespace moe {

namespace {

constexpr int kRExperts = 16;  // experts per workgroup
constexpr int kRWaves = 4;     // waves splitting a workgroup's K slice

// 32-deep k-steps per wave: all of a wave's loads are in registers at once
// (1 + NTB fragments per step)
constexpr int steps_per_wave(int ntb) { return ntb >= 16 ? 2 : 4; }

template <int NTB>  // token blocks of 16 rows
__global__ __launch_bounds__(256) void router_partial_kernel(const bf16_t* __restrict__ x,
                                                             int T, int H,
                                                             const bf16_t* __restrict__ w,
                                                             int E, int nsplit,
                                                             float* __restrict__ part) {
    __shared__ float red[kRWaves][NTB][4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int eb = blockIdx.x, ks = blockIdx.y;
    const int ns = H / 32;
    const int sa = (int)((int64_t)ks * ns / nsplit), sb = (int)((int64_t)(ks + 1) * ns / nsplit);
    constexpr int kRSteps = steps_per_wave(NTB);
    const int s0 = min(sa + wave * kRSteps, sb), s1 = min(s0 + kRSteps, sb);

    // lane (l16, g4) supplies row l16 and k 8*g4 .. +7 of each 32-deep step;
    // rows past E or T repeat the last row (their sums are never stored)
    const bf16_t* wr = w + (int64_t)min(eb * kRExperts + l16, E - 1) * H + g4 * 8;
    const bf16_t* xr[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) xr[tb] = x + (int64_t)min(tb * 16 + l16, T - 1) * H + g4 * 8;

    f32x4_t acc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // A wave owns at most kRSteps k-steps: all its loads go out at once, so
    // the product waits for one memory latency.  Steps past the wave's range
    // (or past K) load an in-range step and use zeros instead.
    bf16x8_t wf[kRSteps], xf[kRSteps][NTB];
    const bf16x8_t zero = {};
#pragma unroll
    for (int u = 0; u < kRSteps; ++u) {
        const bool ok = s0 + u < s1;
        const int k0 = min(s0 + u, ns - 1) * 32;
        wf[u] = ok ? *(const bf16x8_t*)(wr + k0) : zero;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) xf[u][tb] = ok ? *(const bf16x8_t*)(xr[tb] + k0) : zero;
    }
#pragma unroll
    for (int u = 0; u < kRSteps; ++u)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
            acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], xf[u][tb], acc[tb], 0, 0, 0);
    // acc[tb][j] = sum for expert 4*g4 + j of the block and token 16*tb + l16
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][tb][j][lane] = acc[tb][j];
    __syncthreads();
    float* dst = part + (int64_t)ks * T * E;
    for (int tb = wave; tb < NTB; tb += kRWaves) {
        const int t = tb * 16 + l16;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = eb * kRExperts + 4 * g4 + j;
            if (e >= E) continue;
            float v = red[0][tb][j][lane];
#pragma unroll
            for (int q = 1; q < kRWaves; ++q) v += red[q][tb][j][lane];
            dst[(int64_t)t * E + e] = v;
        }
    }
}

__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part,
                                                            int nsplit, int64_t n, int E,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float v = part[i];
    for (int s = 1; s < nsplit; ++s) v += part[(int64_t)s * n + i];
    if (bias) v += bias[i % E];
    logits[i] = v;
}

// The same in-order sum of the slices, rounded once to bf16, four outputs
// per thread (n a multiple of 4).
__global__ __launch_bounds__(256) void slices_to_bf16_kernel(const float* __restrict__ part,
                                                             int nsplit, int64_t n,
                                                             bf16_t* __restrict__ out) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    f32x4_t v = *(const f32x4_t*)(part + i);
    for (int s = 1; s < nsplit; ++s) {
        const f32x4_t u = *(const f32x4_t*)(part + (int64_t)s * n + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += u[q];
    }
    *(uint2*)(out + i) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// K slices for a batch of ntb token blocks (whole k-steps, at most
// 4 * steps_per_wave(ntb) per slice)
int splits_for(int H, int ntb) {
    const int per = kRWaves * steps_per_wave(ntb);
    return std::max(1, (H / 32 + per - 1) / per);
}

template <int NTB>
void launch_partial(const bf16_t* x, int T, int H, const bf16_t* w, int E, float* part,
                    const float* bias, float* logits, hipStream_t s) {
    const int nsplit = splits_for(H, NTB);
    const dim3 gd((unsigned)((E + kRExperts - 1) / kRExperts), (unsigned)nsplit), bd(256);
    router_partial_kernel<NTB><<<gd, bd, 0, s>>>(x, T, H, w, E, nsplit, part);
    const int64_t n = (int64_t)T * E;
    router_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, nsplit, n, E, bias,
                                                                     logits);
}

}  // namespace

int router_splits(int E, int H) {
    (void)E;
    return splits_for(H, 16);  // the most slices any batch size takes
}

hipError_t launch_router_split(const bf16_t* x, int64_t T, int H, const bf16_t* w, int E,
                               const float* bias, float* part, float* logits, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (T > kRouterSplitMaxT || E > kMaxExperts || H % 32 != 0) return hipErrorInvalidValue;
    const int t = (int)T;
    if (T <= 16) launch_partial<1>(x, t, H, w, E, part, bias, logits, s);
    else if (T <= 32) launch_partial<2>(x, t, H, w, E, part, bias, logits, s);
    else if (T <= 64) launch_partial<4>(x, t, H, w, E, part, bias, logits, s);
    else if (T <= 128) launch_partial<8>(x, t, H, w, E, part, bias, logits, s);
    else launch_partial<16>(x, t, H, w, E, part, bias, logits, s);
    return hipGetLastError();
}

int router_tiled_splits(int64_t T, int E, int H) {
    const int64_t tiles = ((T + 127) / 128) * ((E + 127) / 128);
    if (tiles >= 256) return 1;
    // about two workgroups per CU, at least 8 stages of 64 per slice
    const int64_t by_cus = (512 + tiles - 1) / tiles;
    return (int)std::max<int64_t>(1, std::min<int64_t>(by_cus, (H / 64) / 8));
}

hipError_t launch_router_tiled(const bf16_t* x, int64_t T, int H, const bf16_t* w, int E,
                               const float* bias, float* part, float* logits, hipStream_t s) {
    const int nsplit = router_tiled_splits(T, E, H);
    if (T <= 0 || T > INT32_MAX || nsplit < 2) return hipErrorInvalidValue;
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A = x;
    g.lda = H;
    g.a_div = 1;
    g.B = w;
    g.K = H;
    g.N = E;
    g.M = (int32_t)T;
    g.epi = EPI_F32;
    g.C = part;
    g.ldc = E;
    const hipError_t e = launch_tiled_kslices(g, nsplit, s);
    if (e != hipSuccess) return e;
    const int64_t n = T * E;
    router_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, nsplit, n, E, bias,
                                                                     logits);
    return hipGetLastError();
}

int dense_tiled_splits(int64_t T, int N, int K) {
    const int64_t tiles = ((T + 127) / 128) * ((N + 127) / 128);
    if (tiles >= 384) return 1;
    const int64_t by_cus = (512 + tiles - 1) / tiles;
    return (int)std::max<int64_t>(1, std::min<int64_t>(by_cus, (K / 64) / 8));
}

hipError_t launch_dense_sliced_bf16(const bf16_t* A, int64_t T, int K, const bf16_t* B, int N,
                                    float* part, bf16_t* out, hipStream_t s) {
    const int nsplit = dense_tiled_splits(T, N, K);
    if (T <= 0 || T > INT32_MAX || nsplit < 2 || N % 4 != 0) return hipErrorInvalidValue;
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A = A;
    g.lda = K;
    g.a_div = 1;
    g.B = B;
    g.K = K;
    g.N = N;
    g.M = (int32_t)T;
    g.epi = EPI_F32;
    g.C = part;
    g.ldc = N;
    const hipError_t e = launch_tiled_kslices(g, nsplit, s);
    if (e != hipSuccess) return e;
    const int64_t n = T * N;
    slices_to_bf16_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, s>>>(part, nsplit, n, out);
    return hipGetLastError();
}

size_t dense_part_floats(int64_t max_T, int N, int K) {
    size_t n = 0;
    for (int64_t hi = 128; ; hi += 128) {
        const int64_t t = std::min(hi, max_T);
        if (t <= 0) break;
        const int ks = dense_tiled_splits(t, N, K);
        if (ks > 1) n = std::max(n, (size_t)ks * (size_t)t * (size_t)N);
        if (t == max_T || ks == 1) break;
    }
    return n;
}

size_t router_part_floats(int64_t max_T, int E, int H) {
    size_t n = (size_t)router_splits(E, H) * (size_t)std::min<int64_t>(max_T, kRouterSplitMaxT) *
               (size_t)E;
    // the sliced 128x128 product: slices x T peaks at the top of a band of
    // 128 rows; only grids under 256 tiles (T < 32768) are sliced
    for (int64_t hi = kRouterSplitMaxT + 128; ; hi += 128) {
        const int64_t t = std::min(hi, max_T);
        if (t <= kRouterSplitMaxT) break;
        const int ks = router_tiled_splits(t, E, H);
        if (ks > 1) n = std::max(n, (size_t)ks * (size_t)t * (size_t)E);
        if (t == max_T || ks == 1) break;
    }
    return n;
}

}  // namespace moe
