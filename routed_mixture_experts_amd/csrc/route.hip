// Routing: scoring, grouped top-k, renormalisation, routed scaling.
//
// Follows the native routing chain listed in "vLLM-Ascend Kimi K3 MoE Forward
// Insight", Stage 2 "Select Experts": scoring (softmax, sigmoid or
// square-root-softplus), grouped top-k, correction bias, top-k,
// renormalisation, routed scaling.
//
// One 64-lane wavefront routes one token.  Lane l holds experts
// [l*VPL, (l+1)*VPL).  Every selection round is a wave-wide arg-max over
// (key descending, expert index ascending): DPP moves reduce inside each
// 16-lane row, then the four row winners are read back as scalars, so every
// lane ends each round with the same winner and no LDS or atomics are used.
//
// Keys: the fp32 logit itself when the score map alone decides the order (all
// three maps are strictly increasing; group "max" commutes with them), else
// the score in float64 plus the correction bias, compared in float64.
#include "common.h"

namespace moe {

namespace {

constexpr double kNegInf = -__builtin_inf();
constexpr int kNoIndex = 0x7fffffff;

__device__ __forceinline__ bool ranks_before(double ka, int ia, double kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.  After the four steps every lane of a 16-lane
// row has combined all lanes of that row.
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    long long b = __double_as_longlong(v);
    int lo = dpp_i<CTRL>((int)(b & 0xffffffffll));
    int hi = dpp_i<CTRL>((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
    long long b = __double_as_longlong(v);
    int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
    int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(double& k, int& i) {
    double k2 = dpp_d<CTRL>(k);
    int i2 = dpp_i<CTRL>(i);
    if (ranks_before(k2, i2, k, i)) { k = k2; i = i2; }
}

// Wave-wide arg-max; the result is uniform across the wave.
__device__ __forceinline__ void wave_argmax(double& k, int& i) {
    argmax_step<kDppQuadSwap1>(k, i);
    argmax_step<kDppQuadSwap2>(k, i);
    argmax_step<kDppHalfMirror>(k, i);
    argmax_step<kDppMirror>(k, i);
    double bk = readlane_d(k, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        double rk = readlane_d(k, 16 * r);
        int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (ranks_before(rk, ri, bk, bi)) { bk = rk; bi = ri; }
    }
    k = bk;
    i = bi;
}

template <int CTRL>
__device__ __forceinline__ void sum_step(double& v) { v += dpp_d<CTRL>(v); }
template <int CTRL>
__device__ __forceinline__ void max_step(double& v) { v = fmax(v, dpp_d<CTRL>(v)); }

// Wave-wide sum in a fixed tree order (deterministic).
__device__ __forceinline__ double wave_sum(double v) {
    sum_step<kDppQuadSwap1>(v);
    sum_step<kDppQuadSwap2>(v);
    sum_step<kDppHalfMirror>(v);
    sum_step<kDppMirror>(v);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

__device__ __forceinline__ double wave_max(double v) {
    max_step<kDppQuadSwap1>(v);
    max_step<kDppQuadSwap2>(v);
    max_step<kDppHalfMirror>(v);
    max_step<kDppMirror>(v);
    return fmax(fmax(readlane_d(v, 0), readlane_d(v, 16)),
                fmax(readlane_d(v, 32), readlane_d(v, 48)));
}

template <int CTRL>
__device__ __forceinline__ void top2_step(double& a1, double& a2) {
    double b1 = dpp_d<CTRL>(a1), b2 = dpp_d<CTRL>(a2);
    double n1 = fmax(a1, b1);
    double n2 = fmax(fmin(a1, b1), fmax(a2, b2));
    a1 = n1;
    a2 = n2;
}

// Wave-wide two largest values (uniform result).
__device__ __forceinline__ void wave_top2(double& a1, double& a2) {
    top2_step<kDppQuadSwap1>(a1, a2);
    top2_step<kDppQuadSwap2>(a1, a2);
    top2_step<kDppHalfMirror>(a1, a2);
    top2_step<kDppMirror>(a1, a2);
    double b1 = readlane_d(a1, 0), b2 = readlane_d(a2, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        double c1 = readlane_d(a1, 16 * r), c2 = readlane_d(a2, 16 * r);
        double n1 = fmax(b1, c1);
        double n2 = fmax(fmin(b1, c1), fmax(b2, c2));
        b1 = n1;
        b2 = n2;
    }
    a1 = b1;
    a2 = b2;
}

// Score maps in float64.  softplus(v) = max(v,0) + log1p(exp(-|v|)).
__device__ __forceinline__ double score_of(int fn, double l, double smax, double ssum) {
    if (fn == 0) return exp(l - smax) / ssum;
    if (fn == 1) return 1.0 / (1.0 + exp(-l));
    return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;  // uniform per wave
    const int E = a.E;
    const float* lrow = a.logits + t * (int64_t)E;

    float lg[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int e = lane * VPL + i;
        lg[i] = e < E ? lrow[e] : 0.0f;
    }

    // softmax statistics over all E experts.  With renormalisation and the
    // logits as keys they cancel: w_j = exp(l_j - m) / sum_sel exp(l_i - m)
    // with m the largest logit, which is the first selected key.
    const bool sel_softmax = a.score == 0 && a.raw_keys && a.renormalize;
    double smax = 0.0, ssum = 1.0;
    if (a.score == 0 && !sel_softmax) {
        double m = kNegInf;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane * VPL + i < E) m = fmax(m, (double)lg[i]);
        smax = wave_max(m);
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane * VPL + i < E) s += exp((double)lg[i] - smax);
        ssum = wave_sum(s);
    }

    double key[VPL];
    uint32_t elig = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int e = lane * VPL + i;
        if (e < E) {
            elig |= 1u << i;
            if (a.raw_keys) {
                key[i] = (double)lg[i];
            } else {
                double s = score_of(a.score, (double)lg[i], smax, ssum);
                key[i] = a.bias ? s + (double)a.bias[e] : s;
            }
        } else {
            key[i] = kNegInf;
        }
    }

    if (a.G > 1) {
        const int per = E / a.G;
        double gs_lane = kNegInf;  // lane g keeps group g's score
        // lanes per group: when a group fills a power-of-two run of whole
        // lanes (<= 16, inside one DPP row), one segmented top-2 reduction
        // scores every group at once; lane g then fetches group g's score
        // from the group's first lane.  The two best values are the same as
        // the per-group wave reductions below produce.
        const int lpg = per % VPL == 0 ? per / VPL : 0;
        if (lpg == 1 || lpg == 2 || lpg == 4 || lpg == 8 || lpg == 16) {
            double b1 = kNegInf, b2 = kNegInf;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                if (lane * VPL + i < E) {
                    const double v = key[i];
                    if (v > b1) { b2 = b1; b1 = v; }
                    else if (v > b2) { b2 = v; }
                }
            }
            if (lpg >= 2) top2_step<kDppQuadSwap1>(b1, b2);
            if (lpg >= 4) top2_step<kDppQuadSwap2>(b1, b2);
            if (lpg >= 8) top2_step<kDppHalfMirror>(b1, b2);
            if (lpg >= 16) top2_step<kDppMirror>(b1, b2);
            const double gsc = a.group_score == 0 ? b1 : b1 + b2;
            const double mine = __shfl(gsc, min(lane * lpg, 63));
            if (lane < a.G) gs_lane = mine;
        } else
        for (int g = 0; g < a.G; ++g) {
            double b1 = kNegInf, b2 = kNegInf;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                int e = lane * VPL + i;
                if (e < E && e / per == g) {
                    double v = key[i];
                    if (v > b1) { b2 = b1; b1 = v; }
                    else if (v > b2) { b2 = v; }
                }
            }
            wave_top2(b1, b2);
            double gsc = a.group_score == 0 ? b1 : b1 + b2;
            if (lane == g) gs_lane = gsc;
        }
        uint64_t kept = 0;
        for (int r = 0; r < a.topk_group; ++r) {
            bool cand = lane < a.G && !((kept >> lane) & 1ull);
            double ck = cand ? gs_lane : kNegInf;
            int ci = cand ? lane : kNoIndex;
            wave_argmax(ck, ci);
            if (ci < a.G) kept |= 1ull << ci;
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int e = lane * VPL + i;
            if (e < E && !((kept >> (e / per)) & 1ull)) elig &= ~(1u << i);
        }
    }

    int my_id = 0;
    double top_key = 0.0;  // the first (largest) selected key
    for (int j = 0; j < a.k; ++j) {
        double bk = kNegInf;
        int bi = kNoIndex;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int e = lane * VPL + i;
            if (((elig >> i) & 1u) && ranks_before(key[i], e, bk, bi)) { bk = key[i]; bi = e; }
        }
        wave_argmax(bk, bi);
        if (j == 0) top_key = bk;
        if (bi / VPL == lane) elig &= ~(1u << (bi - lane * VPL));
        if (lane == j) my_id = bi;
    }

    // Finite logits always leave k eligible experts; the clamp only keeps a
    // violated precondition (NaN logits) from reading outside the row.
    my_id = min(max(my_id, 0), E - 1);
    double s = 0.0;
    if (lane < a.k)
        s = sel_softmax ? exp((double)lrow[my_id] - top_key)
                        : score_of(a.score, (double)lrow[my_id], smax, ssum);
    double tot = wave_sum(s);
    double w = a.renormalize ? s / tot : s;
    w *= (double)a.scaling;
    if (lane < a.k) {
        a.ids[t * a.k + lane] = my_id;
        a.weights[t * a.k + lane] = (float)w;
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    dim3 grid((unsigned)((a.T + 3) / 4)), block(256);
    if (a.E <= 64) route_kernel<1><<<grid, block, 0, s>>>(a);
    else if (a.E <= 128) route_kernel<2><<<grid, block, 0, s>>>(a);
    else if (a.E <= 256) route_kernel<4><<<grid, block, 0, s>>>(a);
    else if (a.E <= 512) route_kernel<8><<<grid, block, 0, s>>>(a);
    else route_kernel<16><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
