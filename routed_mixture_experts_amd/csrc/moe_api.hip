// C ABI of the routed-MoE forward: host-side validation, workspace layout and
// the launch sequence.  See include/moe.h for the contract of every call.
//
// The stage order is the one of the pages' forward skeleton
// ("vLLM-Ascend Kimi K3 MoE Forward Insight": select_experts, then
// MoECommMethod.fused_experts = dispatch -> unified_apply_mlp -> combine, with
// shared experts beside it) and of the latent runner
// ("vllm.models.kimi_k3.nvidia.latent_moe_runner", _fused_forward: routed input
// transform, experts, tail = RMSNorm -> up-projection -> + shared output).
// Everything is enqueued on the caller's stream; nothing waits on the host.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "permute.h"
#include "router.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

static_assert(MOE_ACT_SILU == ACT_SILU && MOE_ACT_GELU == ACT_GELU &&
                  MOE_ACT_GELU_TANH == ACT_GELU_TANH && MOE_ACT_SWIGLU_CLIP == ACT_SWIGLU_CLIP,
              "activation codes of the ABI and the kernels agree");

// Bump allocator over the caller's workspace.  With base == nullptr it only
// measures, so sizing and carving share one code path.
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base((char*)b) {}
    template <class T>
    T* take(size_t n) {
        off = (off + kAlign - 1) / kAlign * kAlign;
        T* p = base ? (T*)(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
};

size_t elem_size(moe_dtype_t dt) { return dt == MOE_DTYPE_F32 ? 4 : 2; }

bool bad_dtype(moe_dtype_t dt) { return dt != MOE_DTYPE_F32 && dt != MOE_DTYPE_BF16; }

moe_status_t check_cfg(const moe_route_cfg_t* c) {
    if (!c) return MOE_EINVAL;
    const int E = c->num_experts, k = c->top_k, G = c->num_groups;
    if (E < 1 || k < 1 || G < 1 || c->topk_group < 1) return MOE_EINVAL;
    if (E > kMaxExperts || k > kMaxTopK || G > kMaxGroups) return MOE_ENOTSUP;
    if (k > E || E % G != 0 || c->topk_group > G) return MOE_EINVAL;
    if ((int64_t)c->topk_group * (E / G) < k) return MOE_EINVAL;
    if (c->score < 0 || c->score > 2) return MOE_EINVAL;
    if (c->group_score < 0 || c->group_score > 1) return MOE_EINVAL;
    if (G > 1 && c->group_score == MOE_GROUP_TOP2SUM && E / G < 2) return MOE_EINVAL;
    return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

#define MOE_TRY(expr)                              \
    do {                                           \
        moe_status_t st__ = (expr);                \
        if (st__ != MOE_OK) return st__;           \
    } while (0)
#define MOE_HIP(expr) MOE_TRY(hip_status(expr))

bool width_ok(int64_t w) { return w > 0 && w % 64 == 0; }

// The GEMM kernels address one operand (activations, one expert's weights,
// the intermediate h) with 32-bit byte offsets.
bool fits_u32(int64_t rows, int64_t cols, moe_dtype_t dt) {
    return rows * cols * (int64_t)elem_size(dt) < ((int64_t)1 << 32);
}

// Experts with few rows (at most split_rows below; in all-small batches
// kStreamMaxRows) stream their weights once through registers
// (gemm_bf16_stream, one tile per expert); larger experts use 256-row LDS
// tiles (gemm_bf16_big).  fp32 layers use 64-row VALU tiles.
constexpr int kBigRows = 256;
constexpr int kF32Rows = 64;
// Quantised expert weights (FP8 codes, MXFP4 codes with their exponents)
// go through the same 256-row tiles, which take the codes into LDS and
// convert them at the fragment read.  The workspace's tile list is sized for
// 128-row tiles, a bound that also covers them.
constexpr int kTiledRows = 128;

// Dense products: stream the weights for small batches, and where 128x128
// tiles would fill under a quarter of the CUs (a router with few outputs:
// 16-row streaming tiles give many more workgroups); otherwise the 256x256
// tile once its grid covers three quarters of the CUs (measured on the
// latent layer: its 224-tile tail 0.109 against 0.158 ms in 128x128 tiles,
// the 128-tile shared gate/up 0.180 against 0.146 ms), else 128x128.
int dense_path(moe_dtype_t dt, int64_t T, int N, int epi) {
    if (dt == MOE_DTYPE_F32) return GEMM_TILED;
    if (T <= 256) return GEMM_STREAM;
    if (((T + 127) / 128) * ((N + 127) / 128) < 64) return GEMM_STREAM;
    const int64_t cols = epi == EPI_SWIGLU ? (N + 127) / 128 : (N + 255) / 256;
    // the 256-row kernel stores 8-column groups and needs N % 64 == 0
    return (N % 64 == 0 && ((T + 255) / 256) * cols >= 192) ? GEMM_BIG : GEMM_TILED;
}

// Where the two chains split in a batch that is not all-small: groups of at
// most this many rows stream their weights, larger ones take 256-row tiles.  With bf16 weights a group of 33..64 rows runs
// faster in one 256-row tile (each weight byte read once per tile, one or
// two 32-row blocks of MFMAs per wave) than in the streaming kernel, which
// spends four token blocks of LDS reads and MFMAs per weight fragment:
// latent layer (64 rows per group on average) 1.175 against 1.232 ms (then
// with 16-wave streaming workgroups), prefill and grouped layers unchanged.  With FP8 codes
// the same move costs the prefill layer 10.16 against 9.50 ms (its down
// product), so quantised weights stream up to 64 rows.
int split_rows(int fmt) { return fmt == WF_BF16 ? 32 : kStreamMaxRows; }
constexpr int kMinSplitRows = 32;

// Upper bounds of the two tile lists: the large-group list holds tiles of
// `rows` rows; the workspace is sized for the smallest tile of the dtype.
// The small-group list holds one tile per group, or two for groups of
// kStreamMaxRows+1 .. 2*kStreamMaxRows rows when a small batch splits them
// (at most P / (kStreamMaxRows + 1) such groups).  The large-group list has
// at most one partly filled tile per group above the split (at most
// P / (kMinSplitRows + 1) groups).
int64_t small_capacity(moe_dtype_t dt, int E) { return dt == MOE_DTYPE_F32 ? 1 : E; }
int64_t small_capacity_split(int64_t P, int E) {
    return E + std::min<int64_t>(E, P / (kStreamMaxRows + 1));
}
// Batches of at most this many tokens (and no placement) put every group in
// the small-group list: a group has at most T rows.
constexpr int64_t kAllSmallMaxT = 2 * kStreamMaxRows;
int64_t big_capacity(moe_dtype_t dt, int64_t P, int E, int rows) {
    if (dt == MOE_DTYPE_F32) return (P + kF32Rows - 1) / kF32Rows + E;
    return (P + rows - 1) / rows + std::min<int64_t>(E, P / (kMinSplitRows + 1)) + 1;
}
int64_t big_capacity_ws(moe_dtype_t dt, int64_t P, int E) {
    return big_capacity(dt, P, E, dt == MOE_DTYPE_F32 ? kF32Rows : kTiledRows);
}

// Routed expert weights as the kernels take them.
struct ExpertWeights {
    int fmt;           // WeightFmt
    const void* w13;
    const void* w2;
    const void* s13;   // FP8: fp32 [E, 2I] row scales; MXFP4: E8M0 [E, 2I, D/32]
    const void* s2;    // FP8: fp32 [E, D]; MXFP4: E8M0 [E, D, I/32]
    int act = ACT_SILU;
    float act_alpha = 0.0f, act_limit = 0.0f;
};

struct ExpertsWs {
    Tile* small_tiles;
    Tile* big_tiles;
    int32_t* counts;   // [0] small tiles, [1] big tiles
    void* h;
};

ExpertsWs carve_experts(Carve& c, moe_dtype_t dt, int64_t max_T, int k, int E, int I) {
    ExpertsWs w;
    const int64_t P = max_T * k;
    w.small_tiles = c.take<Tile>((size_t)(dt == MOE_DTYPE_F32
                                              ? small_capacity(dt, E)
                                              : small_capacity_split(
                                                    std::min(max_T, kAllSmallMaxT) * k, E)));
    w.big_tiles = c.take<Tile>((size_t)big_capacity_ws(dt, P, E));
    w.counts = c.take<int32_t>(2);
    w.h = c.take<char>((size_t)P * I * elem_size(dt));
    return w;
}

GemmArgs gemm_defaults() {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.a_div = 1;
    return g;
}

// The two halves of one grouped product: groups of at most split_rows rows
// (weight streaming) and the rest (256-row MFMA tiles).
// split_P: the batch's pairs when groups above kStreamMaxRows rows were split
// into two small tiles (0: one tile per group).
moe_status_t small_groups_gemm(GemmArgs g, const ExpertsWs& w, int E, hipStream_t s,
                               int64_t split_P = 0) {
    g.tiles = w.small_tiles;
    g.num_tiles = w.counts;
    g.max_tiles = (int32_t)(split_P > 0 ? small_capacity_split(split_P, E)
                                        : small_capacity(MOE_DTYPE_BF16, E));
    g.tile_m = kStreamMaxRows;
    return hip_status(launch_gemm(1, GEMM_STREAM, g, s));
}

// Rows per tile of the large-group list.
int large_rows(moe_dtype_t dt, int fmt) {
    return dt == MOE_DTYPE_F32 ? kF32Rows : kBigRows;
}

moe_status_t large_groups_gemm(moe_dtype_t dt, GemmArgs g, const ExpertsWs& w, int64_t P, int E,
                               hipStream_t s) {
    const bool f32 = dt == MOE_DTYPE_F32;
    const int rows = large_rows(dt, g.b_fmt);
    g.tiles = w.big_tiles;
    g.num_tiles = w.counts + 1;
    g.max_tiles = (int32_t)big_capacity(dt, P, E, rows);
    g.tile_m = rows;
    const int path = f32 ? GEMM_TILED : GEMM_BIG;
    return hip_status(launch_gemm(f32 ? 0 : 1, path, g, s));
}

// Library-owned side streams (default priority) on which the small-group
// chain and the shared expert run beside the caller's stream.  There is one
// per (device, caller stream) pair, with its own fork / join / shared_done
// events, so calls on different caller streams -- from different host
// threads, eagerly or under graph capture -- never wait on each other's
// events or pull each other's work into a capture.  Calls on one caller
// stream are ordered by that stream, as any work on it is.  The table holds
// kMaxSideCtx pairs per device; past that (or if creating one fails, e.g.
// under a capture mode that forbids it) a call runs unsplit on the caller's
// stream, which gives the same results.
struct SideStream {
    hipStream_t caller = nullptr;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    hipEvent_t shared_done = nullptr;  // the shared expert's products (forward)
};
constexpr int kMaxDevices = 64;
constexpr int kMaxSideCtx = 32;
struct DeviceSides {
    SideStream ctx[kMaxSideCtx];
    int n = 0;
};
std::mutex g_side_mu;  // guards the table only; launches happen outside it
DeviceSides g_side[kMaxDevices];

// The side stream of `caller` on the current device, or nullptr (run
// unsplit).  Entries are never removed, so the pointer stays valid.
SideStream* side_stream(hipStream_t caller) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_side_mu);
    DeviceSides& d = g_side[dev];
    for (int i = 0; i < d.n; ++i)
        if (d.ctx[i].caller == caller) return &d.ctx[i];
    if (d.n == kMaxSideCtx) return nullptr;
    SideStream ss;
    ss.caller = caller;
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.shared_done, hipEventDisableTiming) != hipSuccess ||
        hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) {
        if (ss.fork) (void)hipEventDestroy(ss.fork);
        if (ss.join) (void)hipEventDestroy(ss.join);
        if (ss.shared_done) (void)hipEventDestroy(ss.shared_done);
        (void)hipGetLastError();
        return nullptr;
    }
    d.ctx[d.n] = ss;
    return &d.ctx[d.n++];
}

// Grouped gate/up + SwiGLU, then grouped down, over expert-sorted rows.
//
// When groups average at least kOverlapMinRows rows (prefill-like batches)
// the small groups' chain (gate/up, then down: HBM-bound weight streaming)
// runs on the side stream while the large groups' chain (MFMA-bound) runs on
// the caller's stream; the two touch disjoint rows of h and y_rows.  The
// GEMM1 stage then ends when the large groups' gate/up product ends, and
// GEMM2 covers the rest of both chains.
constexpr int64_t kOverlapMinRows = 16;

// tiles_built: the tile lists in w already match offsets (the forward's
// permute writes them); all_small: it put every group in the small-group
// list, so the large-group products are not launched.
moe_status_t run_experts(moe_dtype_t dt, int64_t T, int k, int E, int D, int I, const void* x,
                         const int32_t* offsets, const int32_t* row_to_pair,
                         const ExpertWeights& ew, void* y_rows, int y_epi, const ExpertsWs& w,
                         hipStream_t s, hipEvent_t* ev, bool tiles_built = false,
                         bool all_small = false, bool side_ok = true) {
    const int64_t P = T * k;
    const bool f32 = dt == MOE_DTYPE_F32;
    if (!tiles_built)
        MOE_HIP(launch_build_tiles(offsets, E,
                                   f32 ? 0 : all_small ? kStreamMaxRows : split_rows(ew.fmt),
                                   large_rows(dt, ew.fmt),
                                   w.small_tiles, w.counts, w.big_tiles, w.counts + 1, s));
    if (ev) MOE_HIP(hipEventRecord(ev[2 * MOE_STAGE_GEMM1], s));

    GemmArgs g1 = gemm_defaults();
    g1.A = x;
    g1.lda = D;
    g1.a_map = row_to_pair;
    g1.a_div = k;
    g1.B = ew.w13;
    g1.b_gstride = (int64_t)2 * I * D;
    g1.b_fmt = ew.fmt;
    g1.b_scale = ew.s13;
    g1.b_scale_gstride = ew.fmt == WF_MXFP4 ? (int64_t)2 * I * (D / 32) : (int64_t)2 * I;
    g1.act = ew.act;
    g1.act_alpha = ew.act_alpha;
    g1.act_limit = ew.act_limit;
    g1.K = D;
    g1.N = I;
    g1.epi = EPI_SWIGLU;
    g1.C = w.h;
    g1.ldc = I;

    GemmArgs g2 = gemm_defaults();
    g2.A = w.h;
    g2.lda = I;
    g2.B = ew.w2;
    g2.b_gstride = (int64_t)D * I;
    g2.b_fmt = ew.fmt;
    g2.b_scale = ew.s2;
    g2.b_scale_gstride = ew.fmt == WF_MXFP4 ? (int64_t)D * (I / 32) : D;
    g2.K = I;
    g2.N = D;
    g2.epi = y_epi;
    g2.C = y_rows;
    g2.ldc = D;

    const auto stage_mark = [&](int stage, int end) -> moe_status_t {
        if (ev) MOE_HIP(hipEventRecord(ev[2 * stage + end], s));
        return MOE_OK;
    };
    if (all_small) {
        // every group is in the small-group list (split into two tiles above
        // kStreamMaxRows rows): no large-group launches, one stream
        MOE_TRY(small_groups_gemm(g1, w, E, s, P));
        MOE_TRY(stage_mark(MOE_STAGE_GEMM1, 1));
        MOE_TRY(stage_mark(MOE_STAGE_GEMM2, 0));
        MOE_TRY(small_groups_gemm(g2, w, E, s, P));
        return stage_mark(MOE_STAGE_GEMM2, 1);
    }
    if (!f32 && P >= kOverlapMinRows * E) {
        SideStream* ss = side_ok ? side_stream(s) : nullptr;
        hipStream_t sc = s;  // the small-group chain's stream
        if (ss) {
            MOE_HIP(hipEventRecord(ss->fork, s));
            MOE_HIP(hipStreamWaitEvent(ss->s, ss->fork, 0));
            sc = ss->s;
        }
        moe_status_t st = small_groups_gemm(g1, w, E, sc);
        if (st == MOE_OK) st = small_groups_gemm(g2, w, E, sc);
        // the caller's stream joins the side stream even after an error
        const moe_status_t sj = ss ? hip_status(hipEventRecord(ss->join, ss->s)) : MOE_OK;
        if (st == MOE_OK) st = large_groups_gemm(dt, g1, w, P, E, s);
        if (st == MOE_OK) st = stage_mark(MOE_STAGE_GEMM1, 1);
        if (st == MOE_OK) st = stage_mark(MOE_STAGE_GEMM2, 0);
        if (st == MOE_OK) st = large_groups_gemm(dt, g2, w, P, E, s);
        if (ss && sj == MOE_OK) MOE_HIP(hipStreamWaitEvent(s, ss->join, 0));
        MOE_TRY(sj);
        MOE_TRY(st);
        return stage_mark(MOE_STAGE_GEMM2, 1);
    }
    if (!f32) MOE_TRY(small_groups_gemm(g1, w, E, s));
    MOE_TRY(large_groups_gemm(dt, g1, w, P, E, s));
    MOE_TRY(stage_mark(MOE_STAGE_GEMM1, 1));
    MOE_TRY(stage_mark(MOE_STAGE_GEMM2, 0));
    if (!f32) MOE_TRY(small_groups_gemm(g2, w, E, s));
    MOE_TRY(large_groups_gemm(dt, g2, w, P, E, s));
    return stage_mark(MOE_STAGE_GEMM2, 1);
}

// Dense C = A . B^T (+ A2 . B2^T) over T rows.
moe_status_t dense_gemm(moe_dtype_t dt, int64_t T, const void* A, int64_t lda, const void* B,
                        int K, const void* A2, int64_t lda2, const void* B2, int K2, int N,
                        int epi, void* C, int64_t ldc, const float* bias, hipStream_t s) {
    GemmArgs g = gemm_defaults();
    g.A = A;
    g.lda = lda;
    g.B = B;
    g.K = K;
    g.A2 = A2;
    g.lda2 = lda2;
    g.B2 = B2;
    g.K2 = A2 ? K2 : 0;
    g.N = N;
    g.M = (int32_t)T;
    g.epi = epi;
    g.C = C;
    g.ldc = ldc;
    g.bias = bias;
    return hip_status(launch_gemm(dt == MOE_DTYPE_F32 ? 0 : 1, dense_path(dt, T, N, epi), g, s));
}

struct ForwardWs {
    float* logits;
    int32_t* ids;
    float* weights;
    int32_t* counts;
    int32_t* offsets;
    int32_t* r2p;
    int32_t* p2r;
    int32_t* chunks;
    ExpertsWs ex;
    void* y_rows;   // expert outputs [T*k, D]: fp16 in bf16 layers, else f32
    void* z;        // latent input [T, L]
    void* normed;   // latent RMSNorm output [T, L]
    void* h_sh;     // shared intermediate [T, Is]
    float* sh;      // shared output [T, H] (no latent)
    int32_t* phys;  // physical slots of the pairs (with a placement)
    float* rpart;   // K-slice partial router sums (bf16 batches of <= kRouterSplitMaxT)
};

// E: experts the permute and expert stages run over (the physical slots
// when a placement is given).
ForwardWs carve_forward(Carve& c, const moe_route_cfg_t* cfg, moe_dtype_t dt, int64_t max_T,
                        int H, int I, const moe_latent_t* lat, const moe_shared_t* sh,
                        int E, bool placed) {
    ForwardWs w;
    const int k = cfg->top_k;
    const int El = cfg->num_experts;
    const int64_t P = max_T * k;
    const int D = lat ? lat->latent : H;
    const size_t es = elem_size(dt);
    w.logits = c.take<float>((size_t)max_T * El);
    w.ids = c.take<int32_t>((size_t)P);
    w.weights = c.take<float>((size_t)P);
    w.counts = c.take<int32_t>((size_t)E);
    w.offsets = c.take<int32_t>((size_t)E + 1);
    w.r2p = c.take<int32_t>((size_t)P);
    w.p2r = c.take<int32_t>((size_t)P);
    w.chunks = c.take<int32_t>((size_t)permute_chunks(P) * E);
    w.ex = carve_experts(c, dt, max_T, k, E, I);
    w.y_rows = c.take<char>((size_t)P * D * (dt == MOE_DTYPE_BF16 ? 2 : 4));
    w.z = lat ? c.take<char>((size_t)max_T * D * es) : nullptr;
    w.normed = lat ? c.take<char>((size_t)max_T * D * es) : nullptr;
    w.h_sh = sh ? c.take<char>((size_t)max_T * sh->inter * es) : nullptr;
    w.sh = (sh && !lat) ? c.take<float>((size_t)max_T * H) : nullptr;
    w.phys = placed ? c.take<int32_t>((size_t)P) : nullptr;
    // partial sums of the K-sliced products: the router, and the latent
    // down-projection (one after the other, so they share the buffer)
    w.rpart = dt == MOE_DTYPE_BF16
                  ? c.take<float>(std::max(router_part_floats(max_T, El, H),
                                           lat ? dense_part_floats(max_T, D, H) : (size_t)0))
                  : nullptr;
    return w;
}

// Slots the permute and expert stages run over; MOE_OK or the error.
moe_status_t placement_slots(const moe_route_cfg_t* cfg, const moe_placement_t* pl, int* E) {
    *E = cfg->num_experts;
    if (!pl) return MOE_OK;
    if (!pl->log2phy || pl->num_physical < 1) return MOE_EINVAL;
    if (pl->num_physical > kMaxExperts) return MOE_ENOTSUP;
    *E = pl->num_physical;
    return MOE_OK;
}

moe_status_t check_forward_shapes(const moe_route_cfg_t* cfg, moe_dtype_t dt, int64_t T, int H,
                                  int I, const moe_latent_t* lat, const moe_shared_t* sh) {
    MOE_TRY(check_cfg(cfg));
    if (bad_dtype(dt) || T < 0) return MOE_EINVAL;
    if (T * (int64_t)cfg->top_k > INT32_MAX / 2) return MOE_ENOTSUP;
    if (!width_ok(H) || !width_ok(I)) return MOE_ENOTSUP;
    {
        const int64_t D = lat ? lat->latent : H;
        const int64_t P = T * cfg->top_k;
        if (!fits_u32(T, std::max<int64_t>(H, D), dt) || !fits_u32(P, I, dt) ||
            !fits_u32(2 * (int64_t)I, D, dt))
            return MOE_ENOTSUP;
        if (sh && (!fits_u32(T, sh->inter, dt) || !fits_u32(2 * (int64_t)sh->inter, H, dt)))
            return MOE_ENOTSUP;
    }
    if (lat) {
        if (!lat->w_down || !lat->gamma || !lat->w_up) return MOE_EINVAL;
        if (!width_ok(lat->latent) || lat->latent > 8192) return MOE_ENOTSUP;
        if (!(lat->rms_eps >= 0.0f)) return MOE_EINVAL;
    }
    if (sh) {
        if (!sh->w13 || !sh->w2) return MOE_EINVAL;
        if (!width_ok(sh->inter)) return MOE_ENOTSUP;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
        case MOE_ENOTSUP: return "MOE_ENOTSUP: shape not supported by this build";
        case MOE_ENOSPACE: return "MOE_ENOSPACE: workspace too small";
        case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
        default: return "unknown moe_status_t";
    }
}

moe_status_t moe_route(const moe_route_cfg_t* cfg, int64_t T, const float* logits,
                       const float* correction_bias, int32_t* topk_ids, float* topk_weights,
                       void* stream) {
    MOE_TRY(check_cfg(cfg));
    if (T < 0) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_EINVAL;
    RouteArgs a;
    a.T = T;
    a.E = cfg->num_experts;
    a.k = cfg->top_k;
    a.G = cfg->num_groups;
    a.topk_group = cfg->topk_group;
    a.score = cfg->score;
    a.group_score = cfg->group_score;
    a.renormalize = cfg->renormalize != 0;
    a.scaling = cfg->routed_scaling;
    a.raw_keys = !correction_bias && (cfg->num_groups == 1 || cfg->group_score == MOE_GROUP_MAX);
    a.logits = logits;
    a.bias = correction_bias;
    a.ids = topk_ids;
    a.weights = topk_weights;
    return hip_status(launch_route(a, (hipStream_t)stream));
}

size_t moe_permute_workspace(int64_t max_T, int32_t k, int32_t E) {
    if (max_T < 0 || k < 1 || E < 1) return 0;
    Carve c(nullptr);
    c.take<int32_t>((size_t)permute_chunks(max_T * k) * E);
    return c.off;
}

moe_status_t moe_permute(int64_t T, int32_t k, int32_t E, const int32_t* topk_ids,
                         int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_to_pair,
                         int32_t* pair_to_row, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1 || E < 1 || k > E) return MOE_EINVAL;
    if (E > kMaxExperts || k > kMaxTopK) return MOE_ENOTSUP;
    if (T * (int64_t)k > INT32_MAX / 2) return MOE_ENOTSUP;
    if (!expert_counts || !expert_offsets) return MOE_EINVAL;
    if (T > 0 && (!topk_ids || !row_to_pair || !pair_to_row)) return MOE_EINVAL;
    if (ws_bytes < moe_permute_workspace(T, k, E) || (T > 0 && !ws)) return MOE_ENOSPACE;
    // T == 0 still writes zero counts and offsets.
    Carve c(ws);
    int32_t* chunks = c.take<int32_t>((size_t)permute_chunks(T * k) * E);
    return hip_status(launch_permute(T * k, E, topk_ids, expert_counts, expert_offsets,
                                     row_to_pair, pair_to_row, chunks, (hipStream_t)stream));
}

size_t moe_experts_workspace(moe_dtype_t dtype, int64_t max_T, int32_t k, int32_t E, int32_t D,
                             int32_t I) {
    if (bad_dtype(dtype) || max_T < 0 || k < 1 || E < 1 || D < 1 || I < 1) return 0;
    Carve c(nullptr);
    carve_experts(c, dtype, max_T, k, E, I);
    return c.off;
}

}  // extern "C"

namespace {

// Expert weights from the C description; MOE_OK or the error of the entry
// point.
moe_status_t expert_weights(moe_dtype_t dtype, const moe_expert_weights_t* d, ExpertWeights* ew) {
    if (!d) return MOE_EINVAL;
    if (d->format != MOE_WEIGHT_DTYPE && d->format != MOE_WEIGHT_FP8_E4M3 &&
        d->format != MOE_WEIGHT_MXFP4)
        return MOE_EINVAL;
    ew->fmt = d->format == MOE_WEIGHT_FP8_E4M3 ? WF_FP8
              : d->format == MOE_WEIGHT_MXFP4  ? WF_MXFP4
                                               : WF_BF16;
    ew->w13 = d->w13;
    ew->w2 = d->w2;
    ew->s13 = ew->fmt != WF_BF16 ? d->w13_scale : nullptr;
    ew->s2 = ew->fmt != WF_BF16 ? d->w2_scale : nullptr;
    if (d->activation < MOE_ACT_SILU || d->activation > MOE_ACT_SWIGLU_CLIP) return MOE_EINVAL;
    ew->act = d->activation;
    ew->act_alpha = d->act_alpha;
    ew->act_limit = d->act_limit;
    if (ew->act == MOE_ACT_SWIGLU_CLIP && !(d->act_alpha > 0.0f && d->act_limit > 0.0f))
        return MOE_EINVAL;
    if (ew->fmt != WF_BF16 && dtype != MOE_DTYPE_BF16) return MOE_ENOTSUP;
    return MOE_OK;
}

bool weights_present(const ExpertWeights& ew) {
    return ew.w13 && ew.w2 && (ew.fmt == WF_BF16 || (ew.s13 && ew.s2));
}

// MXFP4 weights are read 128 elements (64 bytes, 4 scale blocks) per load
// along both reduction widths.
bool weights_fit(const ExpertWeights& ew, int64_t D, int64_t I) {
    return ew.fmt != WF_MXFP4 || (D % 128 == 0 && I % 128 == 0);
}

moe_status_t experts_impl(moe_dtype_t dtype, int64_t T, int32_t k, int32_t E, int32_t D,
                          int32_t I, const void* x, const int32_t* expert_offsets,
                          const int32_t* row_to_pair, const ExpertWeights& ew, float* y_rows,
                          void* ws, size_t ws_bytes, void* stream) {
    if (bad_dtype(dtype) || T < 0 || k < 1 || E < 1 || k > E) return MOE_EINVAL;
    if (E > kMaxExperts || k > kMaxTopK) return MOE_ENOTSUP;
    if (!width_ok(D) || !width_ok(I) || !weights_fit(ew, D, I)) return MOE_ENOTSUP;
    if (T * (int64_t)k > INT32_MAX / 2) return MOE_ENOTSUP;
    if (!fits_u32(T, D, dtype) || !fits_u32(T * k, I, dtype) || !fits_u32(2 * (int64_t)I, D, dtype))
        return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !row_to_pair || !weights_present(ew) || !y_rows)
        return MOE_EINVAL;
    if (!ws || ws_bytes < moe_experts_workspace(dtype, T, k, E, D, I)) return MOE_ENOSPACE;
    Carve c(ws);
    ExpertsWs w = carve_experts(c, dtype, T, k, E, I);
    return run_experts(dtype, T, k, E, D, I, x, expert_offsets, row_to_pair, ew, y_rows, EPI_F32,
                       w, (hipStream_t)stream, nullptr);
}

}  // namespace

extern "C" {

moe_status_t moe_experts(moe_dtype_t dtype, int64_t T, int32_t k, int32_t E, int32_t D,
                         int32_t I, const void* x, const int32_t* expert_offsets,
                         const int32_t* row_to_pair, const void* w13, const void* w2,
                         float* y_rows, void* ws, size_t ws_bytes, void* stream) {
    const ExpertWeights ew = {WF_BF16, w13, w2, nullptr, nullptr, ACT_SILU, 0.0f, 0.0f};
    return experts_impl(dtype, T, k, E, D, I, x, expert_offsets, row_to_pair, ew, y_rows, ws,
                        ws_bytes, stream);
}

moe_status_t moe_experts_ex(moe_dtype_t dtype, int64_t T, int32_t k, int32_t E, int32_t D,
                            int32_t I, const void* x, const int32_t* expert_offsets,
                            const int32_t* row_to_pair, const moe_expert_weights_t* wd,
                            float* y_rows, void* ws, size_t ws_bytes, void* stream) {
    ExpertWeights ew;
    MOE_TRY(expert_weights(dtype, wd, &ew));
    return experts_impl(dtype, T, k, E, D, I, x, expert_offsets, row_to_pair, ew, y_rows, ws,
                        ws_bytes, stream);
}

moe_status_t moe_combine(moe_dtype_t out_dtype, int64_t T, int32_t k, int32_t D,
                         const float* y_rows, const int32_t* pair_to_row,
                         const float* topk_weights, void* out, void* stream) {
    if (bad_dtype(out_dtype) || T < 0 || k < 1 || D < 1) return MOE_EINVAL;
    if (k > kMaxTopK) return MOE_ENOTSUP;
    if (D % 4 != 0) return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!y_rows || !pair_to_row || !topk_weights || !out) return MOE_EINVAL;
    CombineArgs a;
    memset(&a, 0, sizeof(a));
    a.T = T;
    a.k = k;
    a.D = D;
    a.y_rows = y_rows;
    a.pair_to_row = pair_to_row;
    a.weights = topk_weights;
    a.out_dtype = out_dtype == MOE_DTYPE_F32 ? 0 : 1;
    a.out = out;
    return hip_status(launch_combine(a, (hipStream_t)stream));
}

size_t moe_forward_workspace(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t max_T,
                             int32_t H, int32_t I, const moe_latent_t* latent,
                             const moe_shared_t* shared) {
    return moe_forward_workspace_ex(cfg, dtype, max_T, H, I, latent, shared, nullptr);
}

size_t moe_forward_workspace_ex(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t max_T,
                                int32_t H, int32_t I, const moe_latent_t* latent,
                                const moe_shared_t* shared, const moe_placement_t* placement) {
    if (check_forward_shapes(cfg, dtype, max_T, H, I, latent, shared) != MOE_OK) return 0;
    int E = 0;
    if (placement_slots(cfg, placement, &E) != MOE_OK) return 0;
    Carve c(nullptr);
    carve_forward(c, cfg, dtype, max_T, H, I, latent, shared, std::max(E, cfg->num_experts),
                  placement != nullptr);
    return c.off;
}

moe_status_t moe_log2phy(int64_t T, int32_t k, int32_t num_logical, int32_t num_physical,
                         const int32_t* log2phy, const int32_t* topk_ids, int32_t* phys_ids,
                         void* stream) {
    if (T < 0 || k < 1 || num_logical < 1 || num_physical < 1) return MOE_EINVAL;
    if (num_logical > kMaxExperts || num_physical > kMaxExperts) return MOE_ENOTSUP;
    if (T * (int64_t)k > INT32_MAX / 2) return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!log2phy || !topk_ids || !phys_ids) return MOE_EINVAL;
    return hip_status(launch_log2phy(T * k, topk_ids, log2phy, num_logical, num_physical,
                                     phys_ids, (hipStream_t)stream));
}

moe_status_t moe_load_accumulate(int32_t n, const int32_t* counts, int64_t* load, void* stream) {
    if (n < 0) return MOE_EINVAL;
    if (n == 0) return MOE_OK;
    if (!counts || !load) return MOE_EINVAL;
    return hip_status(launch_load_accumulate(n, counts, load, (hipStream_t)stream));
}

}  // extern "C"

namespace {

moe_status_t forward_impl(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T, int32_t H,
                          int32_t I, const void* x, const void* w_router, const float* router_bias,
                          const float* router_logits, const float* correction_bias,
                          const ExpertWeights& ew, const moe_placement_t* placement,
                          const moe_latent_t* latent, const moe_shared_t* shared, void* out,
                          float* logits_out,
                          int32_t* topk_ids_out, float* topk_weights_out,
                          int32_t* expert_counts_out, void* const* stage_events, void* ws,
                          size_t ws_bytes, void* stream, bool side_ok = true) {
    MOE_TRY(check_forward_shapes(cfg, dtype, T, H, I, latent, shared));
    if (!weights_fit(ew, latent ? latent->latent : H, I)) return MOE_ENOTSUP;
    if (T == 0) return MOE_OK;
    if (!x || !weights_present(ew) || !out) return MOE_EINVAL;
    if (!router_logits && !w_router) return MOE_EINVAL;
    int Es = 0;  // experts the permute and expert stages run over
    MOE_TRY(placement_slots(cfg, placement, &Es));
    if (!ws || ws_bytes < moe_forward_workspace_ex(cfg, dtype, T, H, I, latent, shared, placement))
        return MOE_ENOSPACE;

    hipStream_t s = (hipStream_t)stream;
    hipEvent_t* ev = (hipEvent_t*)stage_events;
    const int E = cfg->num_experts, k = cfg->top_k;
    const int D = latent ? latent->latent : H;
    Carve c(ws);
    ForwardWs w = carve_forward(c, cfg, dtype, T, H, I, latent, shared,
                                std::max(Es, cfg->num_experts), placement != nullptr);
    auto mark = [&](int stage, int end) -> moe_status_t {
        if (!ev) return MOE_OK;
        return hip_status(hipEventRecord(ev[2 * stage + end], s));
    };
    auto skip = [&](int stage) -> moe_status_t {
        MOE_TRY(mark(stage, 0));
        return mark(stage, 1);
    };

    // The shared expert reads only x: in bf16 layers its products run on the
    // library's second stream beside routing, dispatch and the routed
    // experts, and the caller's stream waits for them where they are used.
    SideStream* sh_ss = side_ok && shared && dtype == MOE_DTYPE_BF16 ? side_stream(s) : nullptr;
    // Once the shared products are forked, the caller's stream waits for
    // them on every return path, error returns included, so the side stream
    // is always joined back (a graph capture needs that).
    struct SharedJoin {
        hipStream_t s;
        SideStream* ss = nullptr;
        moe_status_t wait() {
            if (!ss) return MOE_OK;
            SideStream* t = ss;
            ss = nullptr;
            return hip_status(hipStreamWaitEvent(s, t->shared_done, 0));
        }
        ~SharedJoin() { (void)wait(); }
    } sh_join{s};
    if (sh_ss) {
        MOE_HIP(hipEventRecord(sh_ss->fork, s));
        MOE_HIP(hipStreamWaitEvent(sh_ss->s, sh_ss->fork, 0));
        moe_status_t st = dense_gemm(dtype, T, x, H, shared->w13, H, nullptr, 0, nullptr, 0,
                                     shared->inter, EPI_SWIGLU, w.h_sh, shared->inter, nullptr,
                                     sh_ss->s);
        if (st == MOE_OK && !latent)
            st = dense_gemm(dtype, T, w.h_sh, shared->inter, shared->w2, shared->inter, nullptr,
                            0, nullptr, 0, H, EPI_F32, w.sh, H, nullptr, sh_ss->s);
        // recorded even after an error, so the caller's stream never waits
        // on a stale record
        MOE_HIP(hipEventRecord(sh_ss->shared_done, sh_ss->s));
        sh_join.ss = sh_ss;
        MOE_TRY(st);
    }
    auto wait_shared = [&]() -> moe_status_t { return sh_join.wait(); };

    // router logits (fp32 accumulate, fp32 out, + optional bias row)
    const float* logits = router_logits;
    if (!logits) {
        float* lo = logits_out ? logits_out : w.logits;
        MOE_TRY(mark(MOE_STAGE_ROUTER, 0));
        if (dtype == MOE_DTYPE_BF16 && T <= kRouterSplitMaxT) {
            // few tokens: K split over workgroups, slices summed in order
            MOE_HIP(launch_router_split((const bf16_t*)x, T, H, (const bf16_t*)w_router, E,
                                        router_bias, w.rpart, lo, s));
        } else if (dtype == MOE_DTYPE_BF16 && router_tiled_splits(T, E, H) > 1) {
            // a 128x128 grid too small for the chip: K split over slices
            MOE_HIP(launch_router_tiled((const bf16_t*)x, T, H, (const bf16_t*)w_router, E,
                                        router_bias, w.rpart, lo, s));
        } else {
            MOE_TRY(dense_gemm(dtype, T, x, H, w_router, H, nullptr, 0, nullptr, 0, E,
                               EPI_F32_BIAS, lo, E, router_bias, s));
        }
        MOE_TRY(mark(MOE_STAGE_ROUTER, 1));
        logits = lo;
    } else {
        MOE_TRY(skip(MOE_STAGE_ROUTER));
        if (logits_out && logits_out != router_logits)
            MOE_HIP(hipMemcpyAsync(logits_out, router_logits, (size_t)T * E * sizeof(float),
                                   hipMemcpyDeviceToDevice, s));
    }

    // latent down-projection of the routed input
    const void* xin = x;
    if (latent) {
        MOE_TRY(mark(MOE_STAGE_DOWNPROJ, 0));
        if (dtype == MOE_DTYPE_BF16 && T > kRouterSplitMaxT &&
            dense_path(dtype, T, D, EPI_OUT) == GEMM_TILED && dense_tiled_splits(T, D, H) > 1) {
            // a 128x128 grid that leaves CUs idle: K split over slices
            MOE_HIP(launch_dense_sliced_bf16((const bf16_t*)x, T, H,
                                             (const bf16_t*)latent->w_down, D, w.rpart,
                                             (bf16_t*)w.z, s));
        } else {
            MOE_TRY(dense_gemm(dtype, T, x, H, latent->w_down, H, nullptr, 0, nullptr, 0, D,
                               EPI_OUT, w.z, D, nullptr, s));
        }
        MOE_TRY(mark(MOE_STAGE_DOWNPROJ, 1));
        xin = w.z;
    } else {
        MOE_TRY(skip(MOE_STAGE_DOWNPROJ));
    }

    // routing
    int32_t* ids = topk_ids_out ? topk_ids_out : w.ids;
    float* wts = topk_weights_out ? topk_weights_out : w.weights;
    MOE_TRY(mark(MOE_STAGE_ROUTE, 0));
    MOE_TRY(moe_route(cfg, T, logits, correction_bias, ids, wts, stream));
    MOE_TRY(mark(MOE_STAGE_ROUTE, 1));

    // dispatch bookkeeping
    int32_t* counts = expert_counts_out ? expert_counts_out : w.counts;
    // (with a placement: logical ids -> physical slots first; the logical ids
    // stay the routing output, the slots decide which weights run)
    MOE_TRY(mark(MOE_STAGE_PERMUTE, 0));
    const int32_t* disp = ids;
    if (placement) {
        MOE_HIP(launch_log2phy(T * k, ids, placement->log2phy, E, Es, w.phys, s));
        disp = w.phys;
    }
    // the permute also writes the GEMM tile lists; at most kAllSmallMaxT
    // tokens (no placement: a group has at most T rows) every group goes to
    // the small-group list
    const bool all_small = T * k <= kSmallPermutePairs && !placement &&
                           dtype == MOE_DTYPE_BF16 && T <= kAllSmallMaxT;
    MOE_HIP(launch_permute_with_tiles(
        T * k, Es, disp, counts, w.offsets, w.r2p, w.p2r, w.chunks,
        dtype == MOE_DTYPE_F32 ? 0 : all_small ? kStreamMaxRows : split_rows(ew.fmt),
        large_rows(dtype, ew.fmt), all_small,
        w.ex.small_tiles, w.ex.counts, w.ex.big_tiles, w.ex.counts + 1, s));
    if (placement && placement->load)
        MOE_HIP(launch_load_accumulate(Es, counts, placement->load, s));
    MOE_TRY(mark(MOE_STAGE_PERMUTE, 1));

    // routed experts
    MOE_TRY(run_experts(dtype, T, k, Es, D, I, xin, w.offsets, w.r2p, ew, w.y_rows,
                        dtype == MOE_DTYPE_BF16 ? EPI_F16 : EPI_F32, w.ex, s, ev,
                        true, all_small, side_ok));

    // shared expert without a latent tail: its output is the combine addend
    if (shared && !latent && sh_ss) {
        MOE_TRY(skip(MOE_STAGE_SHARED));
        MOE_TRY(wait_shared());
    } else if (shared && !latent) {
        MOE_TRY(mark(MOE_STAGE_SHARED, 0));
        MOE_TRY(dense_gemm(dtype, T, x, H, shared->w13, H, nullptr, 0, nullptr, 0, shared->inter,
                           EPI_SWIGLU, w.h_sh, shared->inter, nullptr, s));
        MOE_TRY(dense_gemm(dtype, T, w.h_sh, shared->inter, shared->w2, shared->inter, nullptr,
                           0, nullptr, 0, H, EPI_F32, w.sh, H, nullptr, s));
        MOE_TRY(mark(MOE_STAGE_SHARED, 1));
    }

    // combine (+ fused RMSNorm when latent, + shared addend otherwise)
    CombineArgs ca;
    memset(&ca, 0, sizeof(ca));
    ca.T = T;
    ca.k = k;
    ca.D = D;
    ca.y_rows = w.y_rows;
    ca.y_f16 = dtype == MOE_DTYPE_BF16;
    ca.pair_to_row = w.p2r;
    ca.weights = wts;
    ca.out_dtype = dtype == MOE_DTYPE_F32 ? 0 : 1;
    if (latent) {
        ca.gamma = latent->gamma;
        ca.eps = latent->rms_eps;
        ca.out = w.normed;
    } else {
        ca.addend = w.sh;
        ca.out = out;
    }
    MOE_TRY(mark(MOE_STAGE_COMBINE, 0));
    MOE_HIP(launch_combine(ca, s));
    MOE_TRY(mark(MOE_STAGE_COMBINE, 1));

    if (latent) {
        if (shared && sh_ss) {
            MOE_TRY(skip(MOE_STAGE_SHARED));
            MOE_TRY(wait_shared());
        } else if (shared) {
            MOE_TRY(mark(MOE_STAGE_SHARED, 0));
            MOE_TRY(dense_gemm(dtype, T, x, H, shared->w13, H, nullptr, 0, nullptr, 0,
                               shared->inter, EPI_SWIGLU, w.h_sh, shared->inter, nullptr, s));
            MOE_TRY(mark(MOE_STAGE_SHARED, 1));
        } else {
            MOE_TRY(skip(MOE_STAGE_SHARED));
        }
        // out = normed . w_up^T (+ h_sh . w2_sh^T): one K-concatenated product,
        // one fp32 sum, one rounding
        MOE_TRY(mark(MOE_STAGE_TAIL, 0));
        MOE_TRY(dense_gemm(dtype, T, w.normed, D, latent->w_up, D, shared ? w.h_sh : nullptr,
                           shared ? shared->inter : 0, shared ? shared->w2 : nullptr,
                           shared ? shared->inter : 0, H, EPI_OUT, out, H, nullptr, s));
        MOE_TRY(mark(MOE_STAGE_TAIL, 1));
    } else {
        if (!shared) MOE_TRY(skip(MOE_STAGE_SHARED));
        MOE_TRY(skip(MOE_STAGE_TAIL));
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_forward(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T, int32_t H,
                         int32_t I, const void* x, const void* w_router, const float* router_bias,
                         const float* router_logits, const float* correction_bias,
                         const void* w13, const void* w2, const moe_latent_t* latent,
                         const moe_shared_t* shared, void* out, float* logits_out,
                         int32_t* topk_ids_out, float* topk_weights_out,
                         int32_t* expert_counts_out, void* const* stage_events, void* ws,
                         size_t ws_bytes, void* stream) {
    const ExpertWeights ew = {WF_BF16, w13, w2, nullptr, nullptr, ACT_SILU, 0.0f, 0.0f};
    return forward_impl(cfg, dtype, T, H, I, x, w_router, router_bias, router_logits,
                        correction_bias, ew, nullptr, latent, shared, out, logits_out,
                        topk_ids_out, topk_weights_out, expert_counts_out, stage_events, ws,
                        ws_bytes, stream);
}

moe_status_t moe_forward_ex(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T, int32_t H,
                            int32_t I, const void* x, const void* w_router,
                            const float* router_bias, const float* router_logits,
                            const float* correction_bias, const moe_expert_weights_t* experts,
                            const moe_placement_t* placement, const moe_latent_t* latent,
                            const moe_shared_t* shared, void* out,
                            float* logits_out, int32_t* topk_ids_out, float* topk_weights_out,
                            int32_t* expert_counts_out, void* const* stage_events, void* ws,
                            size_t ws_bytes, void* stream) {
    MOE_TRY(check_forward_shapes(cfg, dtype, T, H, I, latent, shared));
    ExpertWeights ew;
    MOE_TRY(expert_weights(dtype, experts, &ew));
    return forward_impl(cfg, dtype, T, H, I, x, w_router, router_bias, router_logits,
                        correction_bias, ew, placement, latent, shared, out, logits_out,
                        topk_ids_out, topk_weights_out, expert_counts_out, stage_events, ws,
                        ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------------
// moe_forward_noalloc: moe_forward_ex without a workspace argument.  The
// scratch memory comes from a fixed array in the library's device code,
// whose address on each device is looked up once with that device current.
// ------------------------------------------------------------------------
namespace {

static __device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (nullptr on failure).
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status_t moe_forward_noalloc(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T,
                                 int32_t H, int32_t I, const void* x, const void* w_router,
                                 const float* router_bias, const float* router_logits,
                                 const float* correction_bias,
                                 const moe_expert_weights_t* experts,
                                 const moe_placement_t* placement, const moe_latent_t* latent,
                                 const moe_shared_t* shared, void* out, float* logits_out,
                                 int32_t* topk_ids_out, float* topk_weights_out,
                                 int32_t* expert_counts_out, void* stream) {
    MOE_TRY(check_forward_shapes(cfg, dtype, T, H, I, latent, shared));
    ExpertWeights ew;
    MOE_TRY(expert_weights(dtype, experts, &ew));
    if (T == 0) return MOE_OK;
    // the layer's scratch need at this T, checked before any device call
    const size_t need = moe_forward_workspace_ex(cfg, dtype, T, H, I, latent, shared, placement);
    if (need == 0) return MOE_EINVAL;
    if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ENOSPACE;
    void* ws = scratch_ptr();
    if (!ws) return MOE_EHIP;
    // everything on the caller's stream: no side stream is created
    return forward_impl(cfg, dtype, T, H, I, x, w_router, router_bias, router_logits,
                        correction_bias, ew, placement, latent, shared, out, logits_out,
                        topk_ids_out, topk_weights_out, expert_counts_out, nullptr, ws,
                        MOE_NOALLOC_SCRATCH_BYTES, stream, /*side_ok=*/false);
}

}  // extern "C"
