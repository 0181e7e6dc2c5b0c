"""Shared helpers of the parity tests: conversions between torch tensors and
the oracle's numpy arrays, routing settings in both vocabularies, and the
tolerance checks written out once."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from routed_mixture_experts_amd import RouteConfig
from routed_mixture_experts_amd.synth import Workload

# Float output bars: bf16 layers -- relative L2 <= 1e-2 and max |err| <= 3e-2 * rms(ref);
# fp32 layers -- relative L2 <= 1e-5.
BF16_REL_L2 = 1e-2
BF16_MAX_ABS_OVER_RMS = 3e-2
F32_REL_L2 = 1e-5
WEIGHT_ATOL = 1e-6


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a torch tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().to(torch.float64).cpu().numpy()


def npi(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def oracle_cfg(w: Workload) -> O.RouteCfg:
    return O.RouteCfg(num_experts=w.E, top_k=w.k, num_groups=w.num_groups,
                      topk_group=w.topk_group, score=w.score, group_score=w.group_score,
                      renormalize=w.renormalize, routed_scaling=w.routed_scaling)


def lib_cfg(w: Workload) -> RouteConfig:
    return RouteConfig(num_experts=w.E, top_k=w.k, num_groups=w.num_groups,
                       topk_group=w.topk_group, score=w.score, group_score=w.group_score,
                       renormalize=w.renormalize, routed_scaling=w.routed_scaling)


class ExpertFetch:
    """w[e] -> expert e's matrix as float64 numpy, copied from the device one
    expert at a time (the full weight tensor can be tens of GB)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return self.t[int(e)].to(torch.float64).cpu().numpy()


class ExpertFetchFP8:
    """w[e] -> expert e's weights decoded by the oracle from its FP8 E4M3
    codes and row scales (copied from the device one expert at a time)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        self.codes, self.scales = codes, scales

    def __getitem__(self, e):
        e = int(e)
        return O.dequantize_rows(self.codes[e].cpu().numpy(), self.scales[e].cpu().numpy())


class ExpertFetchMXFP4:
    """w[e] -> expert e's weights decoded by the oracle from its MXFP4 codes
    and E8M0 block exponents (copied from the device one expert at a time)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        self.codes, self.scales = codes, scales

    def __getitem__(self, e):
        e = int(e)
        return O.dequantize_mxfp4(self.codes[e].cpu().numpy(), self.scales[e].cpu().numpy())


def latent_np(inp: dict, w: Workload):
    if not w.latent:
        return None
    return dict(w_down=np64(inp["w_down"]), gamma=np64(inp["gamma"]),
                w_up=np64(inp["w_up"]), eps=w.rms_eps)


def shared_np(inp: dict, w: Workload):
    if not w.shared_inter:
        return None
    return dict(w13=np64(inp["w13_sh"]), w2=np64(inp["w2_sh"]))


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def check_float(gpu: np.ndarray, ref: np.ndarray, is_bf16: bool, what: str = "out"):
    """The float bar, printed next to the unavoidable bf16 rounding floor."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = gpu - ref
    rms = float(np.sqrt(np.mean(ref * ref)))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(err).max() / max(rms, 1e-300)) if err.size else 0.0
    if is_bf16:
        floor = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy() - ref
        fl = float(np.abs(floor).max() / max(rms, 1e-300)) if err.size else 0.0
        log(f"[{what}] rel_l2={rel:.3e} (bar {BF16_REL_L2}) max_abs/rms={mx:.3e} "
            f"(bar {BF16_MAX_ABS_OVER_RMS}, bf16 rounding floor {fl:.3e}) n={ref.size}")
        assert rel <= BF16_REL_L2, (what, rel)
        assert mx <= BF16_MAX_ABS_OVER_RMS, (what, mx)
    else:
        log(f"[{what}] rel_l2={rel:.3e} (bar {F32_REL_L2}) n={ref.size}")
        assert rel <= F32_REL_L2, (what, rel)


def check_ids_allowing_near_ties(gpu_ids: np.ndarray, ref_ids: np.ndarray, keys: np.ndarray,
                                 eps: float):
    """Ids must match exactly, except where the oracle's keys of the two
    experts in a differing slot lie within ``eps`` of each other (routing
    there depends on the last bits of a float product, so both answers are
    valid).  Returns the mask of tokens that matched exactly."""
    T, k = ref_ids.shape
    same = (gpu_ids == ref_ids).all(axis=1)
    for t in np.nonzero(~same)[0]:
        assert len(set(gpu_ids[t].tolist())) == k, f"token {t}: repeated expert {gpu_ids[t]}"
        for j in np.nonzero(gpu_ids[t] != ref_ids[t])[0]:
            gap = abs(keys[t, gpu_ids[t, j]] - keys[t, ref_ids[t, j]])
            assert gap <= eps, (f"token {t} slot {j}: ids {gpu_ids[t]} vs {ref_ids[t]}, "
                                f"key gap {gap:.3e} > {eps:.1e}")
    return same


def full_layer_parity(w: Workload, inp: dict, res: dict, w13f, w2f, out_tokens, tag: str,
                      act=None):
    """Parity of a full-size layer run with the GPU's own router product.

    Logits against the oracle's float64 product on every token (relative L2
    <= 1e-5).  The oracle then routes from the GPU's logits, so ids and
    weights must match on every token, and counts, offsets and both maps
    (moe_permute on the GPU ids) bit for bit.  The output is compared element
    by element on ``out_tokens`` (a list, or a function of the oracle's
    counts, offsets and row_to_pair that returns one), which the oracle
    evaluates from the same logits (``w13f`` / ``w2f`` yield one expert's float64 weights at a time)."""
    import routed_mixture_experts_amd as moe
    cfg = oracle_cfg(w)
    corr = None if inp["corr_bias"] is None else np64(inp["corr_bias"])
    lg = np64(res["logits"])
    ref_lg = O.router_logits(np64(inp["x"]), np64(inp["w_router"]),
                             None if inp["router_bias"] is None else np64(inp["router_bias"]))
    rel = float(np.linalg.norm(lg - ref_lg) / np.linalg.norm(ref_lg))
    log(f"[{tag}] logits rel_l2={rel:.2e} (bar 1e-5) over {w.T} tokens")
    assert rel <= 1e-5, rel
    ids, wts, _ = O.route(lg, cfg, corr)
    gids = npi(res["ids"])
    bad = np.nonzero((gids != ids).any(axis=1))[0]
    assert bad.size == 0, f"ids differ on {bad.size} tokens, first {bad[:4]}"
    dw = float(np.abs(np64(res["weights"]) - wts).max())
    assert dw <= WEIGHT_ATOL, dw
    rc, roff, rr2p, rp2r = O.permute(ids, w.E)
    assert (npi(res["counts"]) == rc).all()
    c, off, r2p, p2r = moe.moe_permute(res["ids"], w.E)
    torch.cuda.synchronize()
    assert (npi(c) == rc).all() and (npi(off) == roff).all()
    assert (npi(r2p) == rr2p).all() and (npi(p2r) == rp2r).all()
    log(f"[{tag}] ids, weights (max diff {dw:.1e}), counts, offsets, maps exact over "
        f"{w.T} tokens; load max {rc.max()} min {rc.min()} empty {(rc == 0).sum()}")
    if callable(out_tokens):
        out_tokens = out_tokens(rc, roff, rr2p)
    toks = np.asarray(sorted(set(int(t) for t in out_tokens)), dtype=np.int64)
    ref = O.forward(np64(inp["x"][torch.from_numpy(toks).to(inp["x"].device)]), cfg, w13f, w2f,
                    logits=lg[toks], corr_bias=corr, latent=latent_np(inp, w),
                    shared=shared_np(inp, w), act=act)
    assert (ref["ids"] == ids[toks]).all()
    check_float(np64(res["out"])[toks], ref["out"], w.dtype == "bf16",
                f"{tag} out on {toks.size} tokens")
    return rc, roff, rr2p


def parity_tokens(w: Workload, counts, offsets, row_to_pair, n_random: int = 24, seed: int = 0,
                  big_rows: int = 256, small_max: int = 64, small_block: int = 16,
                  extra_groups: int = 20):
    """Tokens whose outputs a full-size check compares: random ones, the
    first and last token, and for up to ``extra_groups`` groups of each size
    class the token of the group's last row when that row falls in a partly
    filled tile (256-row tiles above ``small_max`` rows, 16-row token blocks
    at or below), plus two tokens of the largest group."""
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(w.T, size=min(n_random, w.T), replace=False).tolist())
    toks |= {0, w.T - 1}
    big = [e for e in range(w.E) if counts[e] > small_max and counts[e] % big_rows]
    small = [e for e in range(w.E) if 0 < counts[e] <= small_max and counts[e] % small_block]
    for grp in (big[:extra_groups], small[:extra_groups]):
        for e in grp:
            toks.add(int(row_to_pair[offsets[e + 1] - 1]) // w.k)
    hot = int(np.argmax(counts))
    for r in (offsets[hot], offsets[hot + 1] - 1):
        toks.add(int(row_to_pair[r]) // w.k)
    return sorted(toks)
