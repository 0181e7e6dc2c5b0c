"""Seeded synthetic inputs for the routed mixture-of-experts workloads.

This module only draws random tensors of the right shapes, dtypes and value
distributions.  It holds none of the layer's arithmetic (no router product, no
scoring, no selection, no expert math), so that both the HIP path and the CPU
oracle can take their inputs from it without sharing any computation.

The workloads are the five shapes the routed-MoE forward is measured on:
a tiny fp32 layer, a decode-sized and a prefill-sized bf16 layer with 384
experts (top-8), a grouped top-k layer with square-root-softplus scoring and a
selection-only correction bias, and a latent layer (down-projection, latent
experts, RMSNorm, up-projection) with a shared expert.  The routing knobs are
the ones the vLLM-Ascend page lists when the runner copies the model's routing
configuration ("Runner Initialization": grouped top-k settings, renormalisation,
scoring function, correction bias, routed scaling).

Recipe (one seed per tensor, base seed 0):
  x:0  router weight:1  w13:2  w2:3  router bias row:4  correction bias:5
  down-proj:6  up-proj:7  shared w13:8  shared w2:9  calibration logits:10
  expert-rank permutation:11  RMSNorm gamma:12
Every weight is N(0, std^2) with std = 1/sqrt(fan_in) (fan_in = the input width
of that matrix) unless the workload fixes it (the tiny layer's router: 0.02).
Activations x ~ N(0, 1).  bf16 tensors are drawn in fp32 and rounded to nearest
even.  The prefill layer's router bias row makes the expert load follow a
Zipf(s) law over a seeded random ranking of the experts; it is calibrated on
simulated i.i.d. N(0,1) logits (a stand-in for the router's output, whose
per-expert logits are close to independent unit normals at this init).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

SEED_X, SEED_WR, SEED_W13, SEED_W2, SEED_BROW, SEED_CORR = 0, 1, 2, 3, 4, 5
SEED_WDN, SEED_WUP, SEED_W13SH, SEED_W2SH, SEED_XCAL, SEED_PERM = 6, 7, 8, 9, 10, 11
SEED_GAMMA = 12


@dataclass(frozen=True)
class Workload:
    """Shapes and routing settings of one routed-MoE layer."""

    name: str
    T: int                      # tokens
    H: int                      # hidden width
    E: int                      # routed experts
    k: int                      # experts per token
    I: int                      # expert SwiGLU intermediate width
    dtype: str = "bf16"         # "bf16" or "f32"
    score: str = "softmax"      # "softmax" | "sigmoid" | "sqrtsoftplus"
    num_groups: int = 1
    topk_group: int = 1
    group_score: str = "max"    # "max" | "top2sum"
    renormalize: bool = True
    routed_scaling: float = 1.0
    router_std: Optional[float] = None   # None: 1/sqrt(H)
    zipf_s: Optional[float] = None       # router bias row giving Zipf(s) load
    corr_bias: Optional[float] = None    # correction bias ~ U(-a, a)
    latent: Optional[int] = None         # latent width L (experts run on it)
    shared_inter: Optional[int] = None   # shared expert intermediate width
    rms_eps: float = 1e-6
    gamma_std: float = 0.0               # RMSNorm gamma = 1 + N(0, gamma_std^2)
    weights: str = "dtype"               # routed expert weights: "dtype" | "fp8_e4m3" | "mxfp4"

    @property
    def D(self) -> int:
        """Width the routed experts read and write (latent if present)."""
        return self.latent if self.latent else self.H

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=64, H=256, E=8, k=2, I=128, dtype="f32",
                          router_std=0.02),
    "decode": Workload("decode", T=128, H=7168, E=384, k=8, I=2048,
                       routed_scaling=2.5),
    "prefill_zipf": Workload("prefill_zipf", T=8192, H=7168, E=384, k=8, I=2048,
                             zipf_s=1.1),
    "grouped_sqrtsoftplus": Workload("grouped_sqrtsoftplus", T=4096, H=4096, E=256,
                                     k=8, I=1536, score="sqrtsoftplus",
                                     num_groups=8, topk_group=4,
                                     group_score="top2sum", corr_bias=0.1),
    "latent_shared": Workload("latent_shared", T=2048, H=7168, E=256, k=8, I=1024,
                              latent=2048, shared_inter=2048),
    # the decode layer with FP8 E4M3 expert weights (one fp32 scale per row)
    "decode_fp8": Workload("decode_fp8", T=128, H=7168, E=384, k=8, I=2048,
                           routed_scaling=2.5, weights="fp8_e4m3"),
    # ... and with MXFP4 expert weights (E2M1 codes, one E8M0 exponent per 32)
    "decode_mxfp4": Workload("decode_mxfp4", T=128, H=7168, E=384, k=8, I=2048,
                             routed_scaling=2.5, weights="mxfp4"),
    # the prefill layer with FP8 E4M3 expert weights
    "prefill_fp8": Workload("prefill_fp8", T=8192, H=7168, E=384, k=8, I=2048,
                            zipf_s=1.1, weights="fp8_e4m3"),
    # ... and with MXFP4 expert weights
    "prefill_mxfp4": Workload("prefill_mxfp4", T=8192, H=7168, E=384, k=8, I=2048,
                              zipf_s=1.1, weights="mxfp4"),
}

FP8_E4M3_MAX = 448.0  # largest finite E4M3 value


def fp8_rows(w: torch.Tensor, chunk: int = 16):
    """FP8 E4M3 codes and per-row scales of a weight tensor [E, n, in].

    scale[e, n] = max|w[e, n, :]| / 448 (1 where the row is all zero) and
    codes = round-to-nearest-even E4M3 encoding of w / scale (torch's
    float8_e4m3fn cast), returned as uint8.  Input construction only: the
    layer and the oracle decode the codes themselves.  Works through ``chunk``
    experts at a time to bound temporary memory."""
    E = w.shape[0]
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    for e0 in range(0, E, chunk):
        blk = w[e0:e0 + chunk].float()
        amax = blk.abs().amax(dim=-1)
        sc = torch.where(amax > 0, amax / FP8_E4M3_MAX, torch.ones_like(amax))
        codes[e0:e0 + chunk] = (blk / sc[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scales[e0:e0 + chunk] = sc
        del blk
    return codes, scales


E2M1_MAX = 6.0  # largest E2M1 magnitude, 1.5 * 2^2
# midpoints between consecutive E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def mxfp4_rows(w: torch.Tensor, chunk: int = 16):
    """MXFP4 codes and E8M0 block exponents of a weight tensor [E, n, in]
    (in a multiple of 32).

    Each block of 32 consecutive inputs of a row gets the exponent x =
    floor(log2(max|w|)) - 2 (so the block maximum lands in [4, 8)), stored as
    the byte s = clamp(x + 127, 1, 254) (127 for an all-zero block).  Each
    w / 2^(s-127) is rounded to the nearest E2M1 magnitude (a tie goes to
    the smaller one, values past 6 saturate at 6) and encoded as sign << 3 |
    magnitude index; element 2j of a row goes to the low nibble of byte j,
    2j + 1 to the high nibble.  Returns (codes [E, n, in/2] uint8, scales
    [E, n, in/32] uint8).  Input construction only: the layer and the oracle
    decode the codes themselves.  Works through ``chunk`` experts at a time
    to bound temporary memory."""
    E, n, K = w.shape
    if K % 32:
        raise ValueError("the input width must be a multiple of 32")
    codes = torch.empty((E, n, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, n, K // 32), dtype=torch.uint8, device=w.device)
    mids = torch.tensor(_E2M1_MIDPOINTS, dtype=torch.float32, device=w.device)
    for e0 in range(0, E, chunk):
        blk = w[e0:e0 + chunk].float().reshape(-1, n, K // 32, 32)
        amax = blk.abs().amax(dim=-1)
        xe = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2.0, torch.zeros_like(amax))
        sb = (xe + 127.0).clamp(1.0, 254.0)
        y = blk / torch.exp2(sb - 127.0)[..., None]
        code = torch.bucketize(y.abs(), mids).to(torch.uint8) | ((y < 0).to(torch.uint8) << 3)
        code = code.reshape(-1, n, K // 2, 2)
        codes[e0:e0 + chunk] = code[..., 0] | (code[..., 1] << 4)
        scales[e0:e0 + chunk] = sb.to(torch.uint8)
        del blk, y, code
    return codes, scales


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, dtype, device, chunk_rows: int = 0) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and rounded to ``dtype``.

    Large tensors are drawn in slabs along dim 0 (``chunk_rows`` rows at a time)
    from one generator stream, so a 34 GB weight never needs an fp32 copy.
    """
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    step = chunk_rows if chunk_rows > 0 else n0
    for s in range(0, n0, step):
        e = min(n0, s + step)
        slab = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device,
                           dtype=torch.float32)
        if std != 1.0:
            slab.mul_(std)
        out[s:e].copy_(slab)
        del slab
    return out


def uniform(shape, a: float, seed: int, device) -> torch.Tensor:
    """U(-a, a) in fp32."""
    g = _gen(seed, device)
    return (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2 - 1) * a


def zipf_router_bias(E: int, k: int, T: int, s: float, iters: int = 60) -> torch.Tensor:
    """Router bias row b[E] (fp32, CPU) that gives a Zipf(s) expert load.

    Expert e gets rank r_e = 1 + perm[e] (seeded permutation, so hot experts are
    scattered) and target load tau_e = min(T*k*r_e^-s / H_{E,s}, 0.999*T).
    The bias is fitted on simulated i.i.d. N(0,1) logits with a damped
    log-count update; it is input construction only.
    """
    perm = torch.randperm(E, generator=_gen(SEED_PERM, "cpu"))
    r = (perm + 1).to(torch.float64)
    harm = float((torch.arange(1, E + 1, dtype=torch.float64) ** (-s)).sum())
    tau = torch.clamp(T * k * r ** (-s) / harm, max=0.999 * T)
    b = -0.55 * torch.log(r)
    sim = torch.randn((T, E), generator=_gen(SEED_XCAL, "cpu"), dtype=torch.float64)
    for _ in range(iters):
        top = torch.topk(sim + b, k, dim=1).indices
        c = torch.bincount(top.reshape(-1), minlength=E).to(torch.float64)
        b = b + 0.5 * (torch.log(tau) - torch.log(c + 0.5))
        b = b - b.mean()
    return b.to(torch.float32)


def make_inputs(w: Workload, device="cpu", chunk_rows: int = 8) -> dict:
    """All tensors of workload ``w`` on ``device``.

    Keys: x[T,H], w_router[E,H], router_bias[E] (fp32) or None,
    corr_bias[E] (fp32) or None, w13[E,2I,D], w2[E,D,I] (for FP8 weights:
    uint8 E4M3 codes plus w13_scale[E,2I], w2_scale[E,D] fp32; for MXFP4
    weights: w13[E,2I,D/2], w2[E,D,I/2] uint8 code pairs plus
    w13_scale[E,2I,D/32], w2_scale[E,D,I/32] uint8 exponents), and for the latent
    layer w_down[L,H], gamma[L], w_up[H,L]; for a shared expert
    w13_sh[2Is,H], w2_sh[H,Is].  Weights are row-major [out, in].
    """
    dt = w.torch_dtype
    D = w.D
    inp = {}
    inp["x"] = normal((w.T, w.H), 1.0, SEED_X, dt, device)
    rstd = w.router_std if w.router_std is not None else 1.0 / math.sqrt(w.H)
    inp["w_router"] = normal((w.E, w.H), rstd, SEED_WR, dt, device)
    inp["router_bias"] = (zipf_router_bias(w.E, w.k, w.T, w.zipf_s).to(device)
                          if w.zipf_s else None)
    inp["corr_bias"] = (uniform((w.E,), w.corr_bias, SEED_CORR, device)
                        if w.corr_bias else None)
    inp["w13"] = normal((w.E, 2 * w.I, D), 1.0 / math.sqrt(D), SEED_W13, dt, device,
                        chunk_rows=chunk_rows)
    inp["w2"] = normal((w.E, D, w.I), 1.0 / math.sqrt(w.I), SEED_W2, dt, device,
                       chunk_rows=chunk_rows)
    if w.weights == "fp8_e4m3":
        # the same draws, quantised per row (the bf16 tensors are dropped)
        for name in ("w13", "w2"):
            codes, scales = fp8_rows(inp[name])
            inp[name] = codes
            inp[name + "_scale"] = scales
    elif w.weights == "mxfp4":
        for name in ("w13", "w2"):
            codes, scales = mxfp4_rows(inp[name])
            inp[name] = codes
            inp[name + "_scale"] = scales
    if w.latent:
        L = w.latent
        inp["w_down"] = normal((L, w.H), 1.0 / math.sqrt(w.H), SEED_WDN, dt, device)
        inp["w_up"] = normal((w.H, L), 1.0 / math.sqrt(L), SEED_WUP, dt, device)
        if w.gamma_std > 0:
            g = normal((L,), w.gamma_std, SEED_GAMMA, torch.float32, device) + 1.0
            inp["gamma"] = g.to(dt)
        else:
            inp["gamma"] = torch.ones((L,), dtype=dt, device=device)
    if w.shared_inter:
        Is = w.shared_inter
        inp["w13_sh"] = normal((2 * Is, w.H), 1.0 / math.sqrt(w.H), SEED_W13SH, dt, device)
        inp["w2_sh"] = normal((w.H, Is), 1.0 / math.sqrt(Is), SEED_W2SH, dt, device)
    return inp


def random_logits(T: int, E: int, seed: int = 0, std: float = 1.0, device="cpu") -> torch.Tensor:
    """Plain fp32 N(0, std^2) logits for exercising the routing stage alone."""
    return torch.randn((T, E), generator=_gen(seed, device), device=device,
                       dtype=torch.float32) * std
