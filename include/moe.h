/*
 * moe.h -- C ABI of the routed mixture-of-experts forward for AMD MI355X (gfx950).
 *
 * The layer follows the routed-MoE pipeline the vLLM-Ascend page traces
 * ("vLLM-Ascend Kimi K3 MoE Forward Insight"): router logits, scoring,
 * grouped top-k with renormalisation and routed scaling (Stage 2, "Select
 * Experts"), dispatch that sorts tokens by expert and returns per-expert token
 * counts, grouped gate/up matmul -> activation -> grouped down matmul, and a
 * combine that restores token order and applies the routing probabilities
 * (Stage 4, "Dispatch, MLP, Combine", AllGather row of the mode table).  The
 * optional latent transform, RMSNorm + up-projection tail and shared expert
 * follow "vllm.models.kimi_k3.nvidia.latent_moe_runner" (LatentMoERunner
 * _fused_forward and the tier-1/tier-2 tails, at tensor-parallel size 1).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller: contiguous,
 *     row-major, at least 16-byte aligned.  Inputs are never written.  The
 *     library allocates, frees and synchronises nothing; scratch memory comes
 *     in as a caller-owned workspace sized from a capacity (max_T), so one
 *     workspace serves every T <= max_T (moe_forward_noalloc instead uses a
 *     fixed scratch array of the library's device code).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are ready when the stream
 *     reaches them.  With buffers and workspace allocated beforehand, a call
 *     can be captured in a HIP graph and replayed: it records no memset, no
 *     host synchronisation and no allocation.
 *   - Weights are [out, in] row-major (the nn.Linear layout).  bf16 values
 *     are IEEE bfloat16 bit patterns (uint16); f32 is IEEE binary32.
 *   - Pair index p = t*k + j names slot j of token t.
 *   - Errors: arguments are validated on the host before anything is
 *     launched; a failed check launches nothing and returns MOE_EINVAL
 *     (inconsistent or null arguments), MOE_ENOTSUP (a shape this build does
 *     not handle: widths not multiples of 64, E > 1024, k > 32, an
 *     activation, intermediate or single-expert weight tensor of 4 GiB or
 *     more) or
 *     MOE_ENOSPACE (workspace too small).  A failed launch returns MOE_EHIP.
 *     T == 0 is valid and launches nothing.  No C++ exception crosses the ABI.
 *   - Preconditions the kernels do not check: logits finite; topk_ids in [0,E).
 *   - Besides moe_forward_noalloc's scratch array (see there), the only
 *     state the library keeps is a table of side streams: for each
 *     (device, caller stream) pair, one stream of its own (default priority,
 *     created on the first call that needs it) with three events (fork,
 *     join, shared expert done).  When a batch splits the experts into many
 *     small and some large groups, the small groups' chain runs there, and
 *     in bf16 layers so does the shared expert; both are forked from and
 *     joined back into `stream` with those events, on every return path
 *     including errors, so a graph capture of `stream` takes them in.
 *     Because each caller stream has its own side stream and events, calls
 *     on different streams may be issued from different host threads, and
 *     one stream may be captured while another runs eagerly.  Calls on one
 *     stream must come from one host thread at a time (as for any work on
 *     one stream).  Past 32 caller streams per device, or if a side stream
 *     cannot be created, a call runs unsplit on `stream` with the same
 *     results.
 */
#ifndef ROUTED_MOE_MI355X_H
#define ROUTED_MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status_t;
enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,
    MOE_ENOTSUP = 2,
    MOE_ENOSPACE = 3,
    MOE_EHIP = 4
};

/* Element type of activations, weights and the layer output. */
typedef int32_t moe_dtype_t;
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

/* Scoring map (page 1, Stage 2: softmax, sigmoid and square-root-softplus). */
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1, MOE_SCORE_SQRTSOFTPLUS = 2 };

/* Group score of grouped top-k: the group's best key, or the sum of its two
 * best keys. */
enum { MOE_GROUP_MAX = 0, MOE_GROUP_TOP2SUM = 1 };

/* Routing settings the runner copies from the model (page 1, "Runner
 * Initialization": grouped top-k settings, renormalisation, scoring function,
 * routed scaling; the correction bias is a tensor argument).
 *   num_experts  E, 1..1024
 *   top_k        k, 1..min(E, 32)
 *   num_groups   G >= 1 dividing E; experts e in [g*E/G, (g+1)*E/G) form group g
 *   topk_group   groups kept, 1..G, with topk_group*E/G >= k
 *   score        MOE_SCORE_*
 *   group_score  MOE_GROUP_* (ignored when G == 1)
 *   renormalize  nonzero: weights are the chosen scores over their sum
 *   routed_scaling  multiplies the final weights                          */
typedef struct {
    int32_t num_experts;
    int32_t top_k;
    int32_t num_groups;
    int32_t topk_group;
    int32_t score;
    int32_t group_score;
    int32_t renormalize;
    float routed_scaling;
} moe_route_cfg_t;

/* Latent transform and tail (page 2, LatentMoERunner): experts run on
 * z = x . w_down^T; the routed output y is normalised as
 * y * rsqrt(mean(y^2) + rms_eps) * gamma and up-projected with w_up^T.
 *   w_down [L, H], gamma [L], w_up [H, L], all in the layer dtype.        */
typedef struct {
    const void* w_down;
    const void* gamma;
    const void* w_up;
    int32_t latent;   /* L */
    float rms_eps;
} moe_latent_t;

/* Shared SwiGLU expert on the original hidden states (page 1, shared experts
 * beside the routed path; page 2, the shared expert receives the
 * untransformed input and its output is added unscaled).
 *   w13 [2*Is, H] (gate rows then up rows), w2 [H, Is], layer dtype.     */
typedef struct {
    const void* w13;
    const void* w2;
    int32_t inter;    /* Is */
} moe_shared_t;

/* ------------------------------------------------------------------------
 * moe_route -- scoring, grouped top-k, renormalisation and routed scaling
 * (page 1, Stage 2 "Select Experts", native chain order).
 *   logits          [T, E] f32, input
 *   correction_bias [E] f32 or NULL; added to the score for selection only
 *   topk_ids        [T, k] int32, output; slot order is descending key,
 *                   ties to the lower expert index (-0.0 == +0.0)
 *   topk_weights    [T, k] f32, output
 * Selection keys are the fp32 logits themselves when no bias is given and the
 * group score is MOE_GROUP_MAX (or G == 1); otherwise the score evaluated in
 * float64 plus the bias, compared in float64.  Weights are computed in
 * float64 and rounded once.  One wavefront per token.
 * ---------------------------------------------------------------------- */
moe_status_t moe_route(const moe_route_cfg_t* cfg, int64_t T, const float* logits,
                       const float* correction_bias, int32_t* topk_ids,
                       float* topk_weights, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute -- stable sort of the T*k (token, slot) pairs by expert
 * (page 1, Stage 4: dispatch sorts tokens by expert and returns expert token
 * counts; Stage 6: the list is per-expert counts or cumulative).
 *   topk_ids       [T, k] int32, input, every id in [0, E)
 *   expert_counts  [E] int32, output
 *   expert_offsets [E+1] int32, output; exclusive prefix sum of the counts
 *   row_to_pair    [T*k] int32, output; row r of the sorted order holds pair
 *                  row_to_pair[r]; inside an expert's rows pairs ascend
 *   pair_to_row    [T*k] int32, output; inverse of row_to_pair
 *   ws, ws_bytes   workspace of at least moe_permute_workspace(max_T, k, E)
 * Deterministic: no atomic operation decides any position.
 * ---------------------------------------------------------------------- */
size_t moe_permute_workspace(int64_t max_T, int32_t k, int32_t E);
moe_status_t moe_permute(int64_t T, int32_t k, int32_t E, const int32_t* topk_ids,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* row_to_pair, int32_t* pair_to_row,
                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_experts -- grouped expert MLP over the expert-sorted rows (page 1,
 * Stage 4: grouped matmul gate/up -> SwiGLU -> grouped matmul down).
 *   x              [T, D] layer dtype; row r of expert e reads token
 *                  row_to_pair[r] / k (gathered, never materialised)
 *   expert_offsets [E+1] int32 from moe_permute
 *   row_to_pair    [T*k] int32 from moe_permute
 *   w13            [E, 2I, D] layer dtype; rows 0..I-1 gate, I..2I-1 up
 *   w2             [E, D, I]  layer dtype
 *   y_rows         [T*k, D] f32, output: expert outputs in sorted-row order,
 *                  kept in fp32 so that combine rounds only once
 *   ws, ws_bytes   at least moe_experts_workspace(dtype, max_T, k, E, D, I)
 * The intermediate h = silu(gate) * up is stored in the layer dtype.
 * D and I must be multiples of 64.
 * ---------------------------------------------------------------------- */
size_t moe_experts_workspace(moe_dtype_t dtype, int64_t max_T, int32_t k, int32_t E,
                             int32_t D, int32_t I);
moe_status_t moe_experts(moe_dtype_t dtype, int64_t T, int32_t k, int32_t E, int32_t D,
                         int32_t I, const void* x, const int32_t* expert_offsets,
                         const int32_t* row_to_pair, const void* w13, const void* w2,
                         float* y_rows, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_combine -- back to token order with the routing weights applied
 * (page 1, Stage 4: combine restores token order and applies probabilities):
 *   out[t] = sum_{j=0..k-1} topk_weights[t,j] * y_rows[pair_to_row[t*k+j]],
 * summed in fp32 in ascending j and rounded once to out_dtype.
 *   y_rows [T*k, D] f32, pair_to_row [T*k] int32, topk_weights [T, k] f32,
 *   out [T, D] in out_dtype.  D must be a multiple of 4.
 * ---------------------------------------------------------------------- */
moe_status_t moe_combine(moe_dtype_t out_dtype, int64_t T, int32_t k, int32_t D,
                         const float* y_rows, const int32_t* pair_to_row,
                         const float* topk_weights, void* out, void* stream);

/* ------------------------------------------------------------------------
 * moe_forward -- the whole layer on one stream (page 2, LatentMoERunner
 * forward(hidden_states, router_logits, ...); page 1, the forward skeleton
 * select_experts -> dispatch -> MLP -> combine, plus shared experts):
 *   [z = x . w_down^T]  -> logits = x . w_router^T (+ router_bias)
 *   -> moe_route -> moe_permute -> moe_experts (on z if latent, else x)
 *   -> combine -> [RMSNorm, . w_up^T] -> [+ shared expert(x)] -> out.
 *   dtype          layer dtype of x, weights and out
 *   T, H, I        tokens, hidden width, routed expert intermediate width
 *   x              [T, H]
 *   w_router       [E, H] layer dtype, or NULL when router_logits is given
 *   router_bias    [E] f32 or NULL: a bias row added to the logits
 *   router_logits  [T, E] f32 or NULL: precomputed logits (skips the router
 *                  product, as the runner's forward takes router_logits)
 *   correction_bias [E] f32 or NULL (selection only)
 *   w13, w2        routed experts as in moe_experts, with D = L if latent
 *                  else H
 *   latent, shared optional (NULL = absent)
 *   out            [T, H] layer dtype, output
 *   logits_out [T,E] f32, topk_ids_out [T,k] int32, topk_weights_out [T,k]
 *   f32, expert_counts_out [E] int32: optional copies of intermediates
 *   (NULL = not wanted)
 *   stage_events   NULL, or 2*MOE_NUM_STAGES hipEvent_t for per-stage
 *                  timing: events[2i] is recorded on `stream` right before
 *                  stage i and events[2i+1] right after it (back to back
 *                  when the stage does not run)
 *   ws, ws_bytes   at least moe_forward_workspace(...) with the same shapes
 * With a shared expert and no latent, out = routed + shared, summed in fp32
 * and rounded once; with a latent, the up-projection and the shared expert's
 * down-projection accumulate into one fp32 sum rounded once.  Between the
 * down product and the combine, the expert rows are kept in fp16 in bf16
 * layers (IEEE binary16: an 11-bit significand, three bits more than bf16,
 * which keeps the output within the bf16 bar) and in fp32 in fp32 layers;
 * the combine sums them in fp32.  Expert outputs must then stay within
 * fp16's finite range, |y| <= 65504 (larger ones become +-inf in `out`).
 * ---------------------------------------------------------------------- */
enum {
    MOE_STAGE_ROUTER = 0,   /* router logits */
    MOE_STAGE_DOWNPROJ,     /* latent down-projection */
    MOE_STAGE_ROUTE,        /* scoring / top-k / weights */
    MOE_STAGE_PERMUTE,      /* counts, offsets, sorted-row maps */
    MOE_STAGE_GEMM1,        /* gate/up + SwiGLU */
    MOE_STAGE_GEMM2,        /* down */
    MOE_STAGE_COMBINE,      /* weighted combine (+ RMSNorm when latent) */
    MOE_STAGE_SHARED,       /* shared expert gate/up + SwiGLU */
    MOE_STAGE_TAIL,         /* up-projection + shared down, or nothing */
    MOE_NUM_STAGES
};

size_t moe_forward_workspace(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t max_T,
                             int32_t H, int32_t I, const moe_latent_t* latent,
                             const moe_shared_t* shared);
moe_status_t moe_forward(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T,
                         int32_t H, int32_t I, const void* x, const void* w_router,
                         const float* router_bias, const float* router_logits,
                         const float* correction_bias, const void* w13, const void* w2,
                         const moe_latent_t* latent, const moe_shared_t* shared,
                         void* out, float* logits_out, int32_t* topk_ids_out,
                         float* topk_weights_out, int32_t* expert_counts_out,
                         void* const* stage_events, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * Expert weights in a storage format other than the layer dtype (page 1,
 * Stage 4: the grouped-matmul paths include W8A8FP and MXFP variants with
 * the dequantisation fused into the grouped matmul).
 *   MOE_WEIGHT_DTYPE     w13 / w2 in the layer dtype, as for moe_experts;
 *                        the scale pointers are ignored.
 *   MOE_WEIGHT_FP8_E4M3  w13 [E, 2I, D] and w2 [E, D, I] hold one OCP e4m3
 *                        code per element (1 sign, 4 exponent bits with
 *                        bias 7, 3 mantissa bits; 0x7F / 0xFF are NaN, there
 *                        is no infinity; largest finite value 448), with one
 *                        fp32 scale per weight row: the expert uses
 *                        W[e, n, :] = decode(codes[e, n, :]) * scale[e, n].
 *                        w13_scale [E, 2I] f32, w2_scale [E, D] f32.  Needs
 *                        layer dtype bf16.  Activations (x, h) stay bf16 and
 *                        every sum is fp32, as in the bf16 layer.
 *   MOE_WEIGHT_MXFP4     OCP microscaling FP4: w13 [E, 2I, D/2] and
 *                        w2 [E, D, I/2] bytes hold two E2M1 codes each
 *                        (element 2j of a row in the low nibble of byte j;
 *                        1 sign, 2 exponent bits with bias 1, 1 mantissa
 *                        bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), and
 *                        every 32 consecutive elements of a row share one
 *                        E8M0 scale byte s, 2^(s - 127): w13_scale
 *                        [E, 2I, D/32] and w2_scale [E, D, I/32] uint8.  The
 *                        expert uses W[e, n, 32b + i] = decode(code) *
 *                        2^(s[e, n, b] - 127).  Scale bytes 0 and 255 (NaN)
 *                        are outside what the kernels handle.  Needs layer
 *                        dtype bf16 and D, I multiples of 128 (MOE_ENOTSUP
 *                        otherwise); activations and sums as for FP8.
 * ---------------------------------------------------------------------- */
typedef enum {
    MOE_WEIGHT_DTYPE = 0,
    MOE_WEIGHT_FP8_E4M3 = 1,
    MOE_WEIGHT_MXFP4 = 2
} moe_weight_format_t;

/* Gate/up activation of the routed experts, h = act(gate, up) (page 1,
 * Stage 4: the activation branches of the grouped MLP; the pages name them
 * without formulas -- these are the readings):
 *   MOE_ACT_SILU        silu(g) * u                       (SwiGLU, default)
 *   MOE_ACT_GELU        0.5 g (1 + erf(g / sqrt 2)) * u
 *   MOE_ACT_GELU_TANH   0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u
 *   MOE_ACT_SWIGLU_CLIP gc * sigmoid(alpha gc) * (uc + 1), gc = min(g, limit),
 *                       uc = clamp(u, -limit, limit): the clipped SwiGLU on
 *                       the gate|up (un-interleaved) row layout; needs
 *                       alpha > 0 and limit > 0 (1.702 and 7 are the usual
 *                       values). */
typedef enum {
    MOE_ACT_SILU = 0,
    MOE_ACT_GELU = 1,
    MOE_ACT_GELU_TANH = 2,
    MOE_ACT_SWIGLU_CLIP = 3
} moe_activation_t;

typedef struct {
    int32_t format;           /* moe_weight_format_t */
    const void* w13;          /* [E, 2I, D] */
    const void* w2;           /* [E, D, I] */
    const void* w13_scale;    /* FP8: [E, 2I] f32; MXFP4: [E, 2I, D/32] u8 */
    const void* w2_scale;     /* FP8: [E, D] f32; MXFP4: [E, D, I/32] u8 */
    int32_t activation;       /* moe_activation_t (0 = SwiGLU) */
    float act_alpha;          /* MOE_ACT_SWIGLU_CLIP only */
    float act_limit;          /* MOE_ACT_SWIGLU_CLIP only */
} moe_expert_weights_t;

/* moe_experts with the expert weights and activation described by `w` (same
 * workspace as moe_experts).  MOE_EINVAL for an unknown format or activation,
 * missing pointers, or clip parameters that are not positive; MOE_ENOTSUP
 * for FP8 or MXFP4 weights with an fp32 layer, and for MXFP4 weights with D
 * or I not a multiple of 128.  A shared expert always uses SwiGLU. */
moe_status_t moe_experts_ex(moe_dtype_t dtype, int64_t T, int32_t k, int32_t E, int32_t D,
                            int32_t I, const void* x, const int32_t* expert_offsets,
                            const int32_t* row_to_pair, const moe_expert_weights_t* w,
                            float* y_rows, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Logical -> physical expert placement and EPLB load (page 1: routing selects
 * logical experts and dispatch may map them through log2phy to physical
 * slots, keeping the router's logical output -- Stage 4, "Runner
 * Initialization"; Stage 6: dispatch's per-expert token counts are added into
 * the layer's moe_load).
 *   num_physical   physical expert slots; the routed expert weights are laid
 *                  out by slot ([num_physical, ...]); a slot holds one
 *                  logical expert's weights (redundant slots hold copies)
 *   log2phy        [num_experts] int32: the slot each logical expert's tokens
 *                  go to; entries in [0, num_physical) (precondition: an
 *                  out-of-range entry is clamped into range, never faults)
 *   load           [num_physical] int64 or NULL: load[s] += tokens sent to
 *                  slot s, once per call
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t num_physical;
    const int32_t* log2phy;
    int64_t* load;
} moe_placement_t;

/* phys_ids[t, j] = log2phy[topk_ids[t, j]] for the T*k pairs. */
moe_status_t moe_log2phy(int64_t T, int32_t k, int32_t num_logical, int32_t num_physical,
                         const int32_t* log2phy, const int32_t* topk_ids, int32_t* phys_ids,
                         void* stream);

/* load[s] += counts[s] for s < n (counts from moe_permute over the slots). */
moe_status_t moe_load_accumulate(int32_t n, const int32_t* counts, int64_t* load,
                                 void* stream);

/* Workspace of moe_forward_ex: as moe_forward_workspace, with the permute and
 * expert stages sized for max(num_experts, placement->num_physical) when a
 * placement is given (NULL: the same as moe_forward_workspace). */
size_t moe_forward_workspace_ex(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t max_T,
                                int32_t H, int32_t I, const moe_latent_t* latent,
                                const moe_shared_t* shared, const moe_placement_t* placement);

/* moe_forward with the routed experts described by `experts` instead of
 * w13 / w2, and an optional placement (NULL: slot = logical id).  With a
 * placement, topk_ids_out keeps the logical ids, the experts run on the slots
 * log2phy gives, expert_counts_out (if given) holds num_physical per-slot
 * counts, and load (if given) accumulates them.  Workspace: at least
 * moe_forward_workspace_ex(...).  Errors as moe_experts_ex; a placement with
 * num_physical outside [1, 1024] or no log2phy is MOE_EINVAL / MOE_ENOTSUP. */
moe_status_t moe_forward_ex(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T,
                            int32_t H, int32_t I, const void* x, const void* w_router,
                            const float* router_bias, const float* router_logits,
                            const float* correction_bias, const moe_expert_weights_t* experts,
                            const moe_placement_t* placement,
                            const moe_latent_t* latent, const moe_shared_t* shared,
                            void* out, float* logits_out, int32_t* topk_ids_out,
                            float* topk_weights_out, int32_t* expert_counts_out,
                            void* const* stage_events, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * moe_forward_noalloc -- moe_forward_ex for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It takes no workspace: its scratch memory is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's device code, which each GPU the
 * library runs on holds until the process ends.  The call allocates nothing
 * (no hipMalloc / hipFree, no side stream: every kernel runs on `stream`);
 * the caller passes inputs and outputs as for moe_forward_ex, which it
 * matches result for result.
 *   Size limit: the layer's scratch need at this T, moe_forward_workspace_ex
 *   (cfg, dtype, T, H, I, latent, shared, placement), must be at most
 *   MOE_NOALLOC_SCRATCH_BYTES (64 MiB: the decode layer with H = 7168,
 *   I = 2048, 384 experts, top-8 fits up to 376 tokens); a larger need
 *   returns MOE_ENOSPACE before anything is launched.
 *   Sharing: every call on one GPU uses that GPU's one array, whatever the
 *   stream or thread, and leaves the last call's contents in it (nothing in
 *   it needs to start at zero).  Calls that overlap in time on one GPU --
 *   two streams, or two host threads -- race on it: order them.
 *   Errors as moe_forward_ex; MOE_EHIP if the array's device address cannot
 *   be obtained.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_noalloc(const moe_route_cfg_t* cfg, moe_dtype_t dtype, int64_t T,
                                 int32_t H, int32_t I, const void* x, const void* w_router,
                                 const float* router_bias, const float* router_logits,
                                 const float* correction_bias,
                                 const moe_expert_weights_t* experts,
                                 const moe_placement_t* placement, const moe_latent_t* latent,
                                 const moe_shared_t* shared, void* out, float* logits_out,
                                 int32_t* topk_ids_out, float* topk_weights_out,
                                 int32_t* expert_counts_out, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* ROUTED_MOE_MI355X_H */
