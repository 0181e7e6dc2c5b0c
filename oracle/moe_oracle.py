"""CPU oracle for the routed mixture-of-experts forward.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path
(the HIP library and its Python binding) never does, and this module imports
nothing from it.

Plain numpy, float64 throughout, written from the step list on the pages:

* "vLLM-Ascend Kimi K3 MoE Forward Insight" (page 1): Stage 2 "Select
  Experts" names the native routing chain in order -- scoring, grouped top-k,
  correction bias, top-k, renormalisation, routed scaling; "Runner
  Initialization" names the routing knobs; Stage 4 "Dispatch, MLP, Combine"
  (its mode table, AllGather row) says dispatch sorts tokens by expert and
  returns per-expert token counts and combine restores token order and applies
  the probabilities; the MLP is grouped gate/up matmul -> activation ->
  grouped down matmul; Stage 6 says the expert-token list may be per-expert
  counts or cumulative.
* "vllm.models.kimi_k3.nvidia.latent_moe_runner" (page 2): ``_fused_forward``
  runs the routed experts on the transformed (latent) input while the shared
  expert sees the original hidden states; the tail reduces the latent, applies
  RMSNorm, up-projects with ``up_proj.weight`` transposed and adds the shared
  output (``_overlap_allreduce_tail``; ``_shard_up_proj_tail`` folds the same
  sum into the GEMM's beta-add); at tensor-parallel size 1,
  ``allreduce_norm_latent_out`` is the plain norm.
* "Kimi K3 三平台架构对比解读" (page 3): the PyTorch fallback of the attention
  residual spells out the RMS convention used here -- fp32 values times
  rsqrt(mean(x^2) + eps).

Readings where the pages are silent (each is listed in the design notes):
selection keys are the raw logits when the score map is monotone and no
correction bias or group sum is involved, else the score evaluated in float64
plus the bias; ties go to the lower expert index and -0.0 equals +0.0; the
group score is the group's best key or the sum of its two best keys; groups
are contiguous; renormalisation divides the unbiased scores of the selected
experts by their sum and routed scaling multiplies afterwards; combine weights
are applied to expert outputs, never to inputs; rows of w13 are gate then up;
rows inside an expert's segment keep ascending pair order p = t*k + j.

The expert activation is SwiGLU unless set otherwise (page 1, Stage 4 also
lists a clipped SwiGLU on the un-interleaved gate|up layout, GELU and
GELU-tanh, without formulas).  Readings: GELU = x * Phi(x) (erf form) and its
tanh approximation, applied as gelu(gate) * up; the clipped SwiGLU is
min(g, L) * sigmoid(alpha * min(g, L)) * (clamp(u, -L, L) + 1), the form of
the published open-weight MLP that names it, with alpha and L as
parameters.

Expert weights may also come as 8-bit floating-point codes (page 1, Stage 4:
the grouped-matmul paths include W8A8FP, W4A8 and MXFP variants with the
dequantisation fused into the matmul; the pages give no format).  Reading:
OCP FP8 E4M3 codes with one fp32 scale per weight row, the expert using
decode(code) * scale; activations and every sum stay as in the unquantised
layer.  For the MXFP variant the reading is the OCP Microscaling MXFP4
format: E2M1 codes (two per byte, element 2j in the low nibble of byte j of
a row) and one E8M0 exponent byte s per 32 consecutive elements of a row,
the weight being decode(code) * 2^(s - 127); activations and sums again as
in the unquantised layer.

Parity pins: every function here is checked in the CPU test suite against
something other than itself (closed forms, brute force over all subsets,
textbook special cases, a dense every-expert reference written with torch).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

f64 = np.float64


@dataclass(frozen=True)
class RouteCfg:
    """Routing settings copied from the model (page 1, "Runner Initialization")."""

    num_experts: int
    top_k: int
    num_groups: int = 1
    topk_group: int = 1
    score: str = "softmax"        # softmax | sigmoid | sqrtsoftplus
    group_score: str = "max"      # max | top2sum
    renormalize: bool = True
    routed_scaling: float = 1.0


# ---------------------------------------------------------------- scoring ---

def softplus(v: np.ndarray) -> np.ndarray:
    """ln(1 + e^v) in float64, written so that it does not overflow."""
    v = np.asarray(v, dtype=f64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def score(logits: np.ndarray, fn: str) -> np.ndarray:
    """Scores s[T,E] from logits (page 1, Stage 2: softmax, sigmoid or
    square-root-softplus scoring), evaluated in float64."""
    l = np.asarray(logits, dtype=f64)
    if fn == "softmax":
        m = l.max(axis=-1, keepdims=True)
        e = np.exp(l - m)
        return e / e.sum(axis=-1, keepdims=True)
    if fn == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    if fn == "sqrtsoftplus":
        return np.sqrt(softplus(l))
    raise ValueError(fn)


def keys_are_raw_logits(cfg: RouteCfg, has_bias: bool) -> bool:
    """True when ordering by score equals ordering by the raw logit.

    All three score maps are strictly increasing in the logit, and a group's
    best key is the image of its best logit, so without a correction bias and
    without a two-key group sum the exact ordering is the ordering of the fp32
    logits themselves (no rounding of exp/log can create false ties)."""
    return (not has_bias) and (cfg.num_groups == 1 or cfg.group_score == "max")


def selection_keys(logits: np.ndarray, cfg: RouteCfg,
                   corr_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-expert selection keys kappa[T,E] (float64).

    The correction bias enters selection only (page 1, Stage 2 lists it
    between grouped top-k and the final top-k; renormalisation later uses the
    unbiased scores)."""
    l = np.asarray(logits, dtype=f64)
    if keys_are_raw_logits(cfg, corr_bias is not None):
        return l.copy()
    s = score(l, cfg.score)
    if corr_bias is not None:
        s = s + np.asarray(corr_bias, dtype=f64)[None, :]
    return s


# -------------------------------------------------------------- selection ---

def _order_desc(keys_row: np.ndarray) -> np.ndarray:
    """Indices sorted by key descending, ties to the lower index.

    numpy compares with '<', so -0.0 and +0.0 are equal keys."""
    idx = np.arange(keys_row.shape[0])
    return np.lexsort((idx, -keys_row))


def group_scores(keys: np.ndarray, cfg: RouteCfg) -> np.ndarray:
    """Group score g[T,G] over contiguous groups of E/G experts: the group's best
    key ("max") or the sum of its two best keys ("top2sum")."""
    T, E = keys.shape
    G = cfg.num_groups
    kg = keys.reshape(T, G, E // G)
    if cfg.group_score == "max":
        return kg.max(axis=-1)
    if cfg.group_score == "top2sum":
        srt = np.sort(kg, axis=-1)
        return srt[..., -1] + srt[..., -2]
    raise ValueError(cfg.group_score)


def select_experts(keys: np.ndarray, cfg: RouteCfg) -> np.ndarray:
    """Grouped top-k (page 1, Stage 2): keep the ``topk_group`` best groups,
    then the k best keys among their experts, in descending key order."""
    T, E = keys.shape
    k = cfg.top_k
    ids = np.empty((T, k), dtype=np.int64)
    allowed = np.ones((T, E), dtype=bool)
    if cfg.num_groups > 1:
        gs = group_scores(keys, cfg)
        per = E // cfg.num_groups
        for t in range(T):
            keep = _order_desc(gs[t])[: cfg.topk_group]
            mask = np.zeros(cfg.num_groups, dtype=bool)
            mask[keep] = True
            allowed[t] = np.repeat(mask, per)
    for t in range(T):
        cand = np.nonzero(allowed[t])[0]
        order = cand[_order_desc(keys[t, cand])]
        ids[t] = order[:k]
    return ids


def route_weights(logits: np.ndarray, ids: np.ndarray, cfg: RouteCfg) -> np.ndarray:
    """Combine weights w[T,k] (float64): unbiased scores of the chosen experts,
    renormalised to sum 1 if asked, then times the routed scaling factor
    (page 1, Stage 2 order: renormalisation, then routed scaling)."""
    s = score(logits, cfg.score)
    w = np.take_along_axis(s, ids, axis=1)
    if cfg.renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w * f64(cfg.routed_scaling)


def route(logits: np.ndarray, cfg: RouteCfg, corr_bias: Optional[np.ndarray] = None):
    """Scoring -> keys -> grouped top-k -> weights.  Returns (ids, weights, keys)."""
    keys = selection_keys(logits, cfg, corr_bias)
    ids = select_experts(keys, cfg)
    w = route_weights(logits, ids, cfg)
    return ids, w, keys


# ---------------------------------------------------------------- permute ---

def permute(ids: np.ndarray, num_experts: int):
    """Sort (token, slot) pairs by expert (page 1, Stage 4, AllGather dispatch:
    sort tokens by expert and return per-expert token counts).

    Pairs are p = t*k + j.  Returns counts[E], offsets[E+1] (exclusive scan --
    the cumulative form of the expert-token list, page 1 Stage 6),
    row_to_pair[P] (stable: ascending p within an expert) and pair_to_row[P]
    (its inverse)."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int64)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_to_pair = np.argsort(flat, kind="stable")
    pair_to_row = np.empty_like(row_to_pair)
    pair_to_row[row_to_pair] = np.arange(flat.shape[0])
    return counts, offsets, row_to_pair, pair_to_row


# ----------------------------------------------------------------- experts ---

def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (the 8-bit floating-point format behind
    page 1's W8A8FP path, per the reading in the header): bit 7 is the sign,
    bits 6..3 the exponent field e with bias 7, bits 2..0 the mantissa m.
    e > 0 gives (1 + m/8) * 2^(e-7); e = 0 gives the subnormal (m/8) * 2^-6;
    e = 15 with m = 7 is NaN (the format has no infinities, so e = 15 with
    m < 7 is an ordinary value, up to 448)."""
    # the formula is evaluated once on all 256 codes; the codes then index
    # that table (the same values, without per-element exp2 on large tensors)
    c = np.arange(256, dtype=np.int64)
    sign, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(sign == 1, -mag, mag)
    table = np.where((e == 15) & (m == 7), np.nan, val).astype(f64)
    return table[np.asarray(codes, dtype=np.uint8)]


def dequantize_rows(codes, scale) -> np.ndarray:
    """Weights from FP8 codes with one scale per row (the last axis is the
    input width): W[..., n, :] = decode(codes[..., n, :]) * scale[..., n]."""
    return fp8_e4m3_decode(codes) * np.asarray(scale, dtype=f64)[..., None]


def e2m1_decode(codes) -> np.ndarray:
    """Values of 4-bit OCP E2M1 codes (the element format of MXFP4, per the
    reading in the header): bit 3 is the sign, bits 2..1 the exponent field e
    with bias 1, bit 0 the mantissa m.  e > 0 gives (1 + m/2) * 2^(e-1); e = 0
    gives the subnormal m/2.  Every code is finite."""
    c = np.arange(16, dtype=np.int64)        # all codes, then a table lookup
    sign, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    table = np.where(sign == 1, -mag, mag).astype(f64)
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.size and codes.max() > 15:
        raise ValueError("E2M1 codes are 4-bit")
    return table[codes]


def e8m0_decode(codes) -> np.ndarray:
    """Values of OCP E8M0 scale bytes: 2^(s - 127); s = 255 is NaN."""
    s = np.arange(256, dtype=np.int64)       # all bytes, then a table lookup
    table = np.where(s == 255, np.nan, np.exp2(s - 127.0)).astype(f64)
    return table[np.asarray(codes, dtype=np.uint8)]


def dequantize_mxfp4(codes, scales) -> np.ndarray:
    """Weights from MXFP4 storage: codes [..., K/2] bytes with element 2j of
    a row in the low nibble of byte j and 2j+1 in the high nibble; scales
    [..., K/32] E8M0 bytes, one per 32 consecutive elements.  Returns
    [..., K] float64: W[..., 32b + i] = e2m1(code) * 2^(s[..., b] - 127)."""
    c = np.asarray(codes, dtype=np.uint8)
    elems = np.stack([c & 15, c >> 4], axis=-1).reshape(*c.shape[:-1], 2 * c.shape[-1])
    sc = e8m0_decode(scales)
    if sc.shape[-1] * 32 != elems.shape[-1]:
        raise ValueError("one scale byte per 32 elements")
    return e2m1_decode(elems) * np.repeat(sc, 32, axis=-1)


def map_to_physical(ids, log2phy) -> np.ndarray:
    """Physical slot of every selected expert (page 1, Stage 4: with dynamic
    placement, dispatch maps the logical topk_ids through log2phy; the
    router's logical output is kept): phys[t, j] = log2phy[ids[t, j]]."""
    return np.asarray(log2phy, dtype=np.int64)[np.asarray(ids, dtype=np.int64)]


def accumulate_load(load, counts) -> np.ndarray:
    """EPLB heat (page 1, Stage 6): the dispatch's per-expert token counts
    are added into the layer's load."""
    return np.asarray(load, dtype=np.int64) + np.asarray(counts, dtype=np.int64)


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def gelu(v: np.ndarray) -> np.ndarray:
    """GELU, x * Phi(x) with the normal CDF written through erf."""
    from scipy.special import erf
    v = np.asarray(v, dtype=f64)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


def gelu_tanh(v: np.ndarray) -> np.ndarray:
    """The tanh approximation of GELU."""
    v = np.asarray(v, dtype=f64)
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)))


def glu(g: np.ndarray, u: np.ndarray, act: Optional[dict] = None) -> np.ndarray:
    """Gate/up activation h = act(gate, up) (page 1, Stage 4 lists SwiGLU, a
    clipped SwiGLU on the un-interleaved gate|up layout, GELU and GELU-tanh
    as the MLP's activation branches; the formulas are the readings in the
    header).  ``act`` = None or dict(kind="silu" | "gelu" | "gelu_tanh" |
    "swiglu_clip", alpha=..., limit=...)."""
    kind = (act or {}).get("kind", "silu")
    if kind == "silu":
        return silu(g) * u
    if kind == "gelu":
        return gelu(g) * u
    if kind == "gelu_tanh":
        return gelu_tanh(g) * u
    if kind == "swiglu_clip":
        alpha, limit = float(act["alpha"]), float(act["limit"])
        gc = np.minimum(g, limit)
        uc = np.clip(u, -limit, limit)
        return gc / (1.0 + np.exp(-alpha * gc)) * (uc + 1.0)
    raise ValueError(kind)


def expert_mlp(X: np.ndarray, w13_e: np.ndarray, w2_e: np.ndarray,
               act: Optional[dict] = None) -> np.ndarray:
    """One expert (page 1, Stage 4: gate/up matmul -> activation -> down
    matmul; SwiGLU unless ``act`` says otherwise, see glu).

    w13_e is [2I, D] with gate rows first, then up rows; w2_e is [D, I]."""
    w13_e = np.asarray(w13_e, dtype=f64)
    w2_e = np.asarray(w2_e, dtype=f64)
    I = w2_e.shape[1]
    gu = np.asarray(X, dtype=f64) @ w13_e.T
    h = glu(gu[:, :I], gu[:, I:], act)
    return h @ w2_e.T


def run_experts(xin: np.ndarray, k: int, offsets: np.ndarray, row_to_pair: np.ndarray,
                w13, w2, act: Optional[dict] = None) -> np.ndarray:
    """Grouped expert MLP over the expert-sorted rows.  Row r of expert e reads
    token row_to_pair[r] // k.  ``w13[e]`` / ``w2[e]`` may be any indexable
    that yields expert e's matrices.  Returns y_rows[P, D] (float64)."""
    xin = np.asarray(xin)
    P = row_to_pair.shape[0]
    E = offsets.shape[0] - 1
    D = xin.shape[1]
    y = np.zeros((P, D), dtype=f64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        X = np.asarray(xin[row_to_pair[a:b] // k], dtype=f64)
        y[a:b] = expert_mlp(X, w13[e], w2[e], act)
    return y


def combine(y_rows: np.ndarray, pair_to_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """Back to token order with the routing weights applied (page 1, Stage 4,
    AllGather combine): out[t] = sum_j w[t,j] * y_rows[pair_to_row[t*k+j]]."""
    T, k = weights.shape
    rows = y_rows[pair_to_row.reshape(T, k)]          # [T, k, D]
    return np.einsum("tk,tkd->td", np.asarray(weights, dtype=f64), rows)


# ------------------------------------------------------ latent + shared tail ---

def rmsnorm(v: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """v * rsqrt(mean(v^2) + eps) * gamma (page 3, fp32 RMS convention of the
    attention-residual fallback; page 2 passes a zero weight bias, i.e. the
    standard gamma, not 1 + gamma)."""
    v = np.asarray(v, dtype=f64)
    inv = 1.0 / np.sqrt((v * v).mean(axis=-1, keepdims=True) + eps)
    return v * inv * np.asarray(gamma, dtype=f64)[None, :]


def shared_expert(x: np.ndarray, w13_sh: np.ndarray, w2_sh: np.ndarray) -> np.ndarray:
    """Shared SwiGLU expert on the original hidden states (page 2,
    ``_fused_forward``: the shared expert receives the untransformed input)."""
    return expert_mlp(x, w13_sh, w2_sh)


# ---------------------------------------------------------------- forward ---

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l = x . W_r^T (+ bias row), float64."""
    l = np.asarray(x, dtype=f64) @ np.asarray(w_router, dtype=f64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, dtype=f64)[None, :]
    return l


def forward(x, cfg: RouteCfg, w13, w2, *, w_router=None, router_bias=None,
            logits=None, corr_bias=None, latent=None, shared=None, act=None) -> dict:
    """The whole routed-MoE forward as a chain of the steps above.

    ``logits`` (if given) replaces the router product, as in the runner's
    ``forward(hidden_states, router_logits, ...)`` signature (page 2).
    ``latent`` = dict(w_down[L,H], gamma[L], w_up[H,L], eps) and
    ``shared`` = dict(w13[2Is,H], w2[H,Is]) add the latent transform and tail
    and the shared expert (page 2).  ``act``: the routed experts' activation
    (see glu; the shared expert is SwiGLU).  Returns every intermediate."""
    x64 = np.asarray(x, dtype=f64)
    if logits is None:
        logits = router_logits(x64, w_router, router_bias)
    logits = np.asarray(logits, dtype=f64)
    k = cfg.top_k
    ids, w, keys = route(logits, cfg, corr_bias)
    counts, offsets, r2p, p2r = permute(ids, cfg.num_experts)
    xin = x64
    if latent is not None:
        xin = x64 @ np.asarray(latent["w_down"], dtype=f64).T
    y_rows = run_experts(xin, k, offsets, r2p, w13, w2, act)
    routed = combine(y_rows, p2r, w)
    res = dict(logits=logits, ids=ids, weights=w, keys=keys, counts=counts,
               offsets=offsets, row_to_pair=r2p, pair_to_row=p2r, y_rows=y_rows,
               routed=routed, xin=xin)
    sh = shared_expert(x64, shared["w13"], shared["w2"]) if shared is not None else None
    if latent is not None:
        r = rmsnorm(routed, latent["gamma"], latent["eps"])
        out = r @ np.asarray(latent["w_up"], dtype=f64).T
        if sh is not None:
            out = out + sh
        res["normed"] = r
    else:
        out = routed if sh is None else routed + sh
    res["shared"] = sh
    res["out"] = out
    return res


def forward_tokens(tokens, x, cfg: RouteCfg, w13, w2, *, w_router=None, router_bias=None,
                   logits=None, corr_bias=None, latent=None, shared=None, act=None) -> dict:
    """The same layer evaluated token by token for a list of tokens, without
    the permute (tokens are independent in a routed MoE).  Used to check
    sampled outputs of very large layers, where ``w13[e]``/``w2[e]`` fetch one
    expert at a time."""
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.asarray(x[tokens], dtype=f64)
    if logits is None:
        lg = router_logits(xs, w_router, router_bias)
    else:
        lg = np.asarray(logits, dtype=f64)[tokens]
    ids, w, keys = route(lg, cfg, corr_bias)
    xin = xs if latent is None else xs @ np.asarray(latent["w_down"], dtype=f64).T
    routed = np.zeros((tokens.shape[0], xin.shape[1]), dtype=f64)
    for i in range(tokens.shape[0]):
        for j in range(cfg.top_k):
            e = int(ids[i, j])
            y = expert_mlp(xin[i:i + 1], w13[e], w2[e], act)[0]
            routed[i] += w[i, j] * y
    sh = shared_expert(xs, shared["w13"], shared["w2"]) if shared is not None else None
    if latent is not None:
        out = rmsnorm(routed, latent["gamma"], latent["eps"]) @ \
            np.asarray(latent["w_up"], dtype=f64).T
        if sh is not None:
            out = out + sh
    else:
        out = routed if sh is None else routed + sh
    return dict(logits=lg, ids=ids, weights=w, keys=keys, routed=routed, out=out)
