"""GPU parity of the MXFP4 expert-weight path (moe_experts_ex, moe_forward_ex)
against the oracle.

The oracle decodes the same E2M1 codes and E8M0 block exponents into float64
weights (oracle.dequantize_mxfp4), so both sides multiply by exactly the same
weight values; the remaining difference is the bf16 rounding of h and of the
output, and the bar is the bf16 layer's.  Shapes cover the streaming kernel
with 1, 2 and 4 token blocks (including passes whose last chunks lie past K),
the 256x256 kernel for groups above 64 rows (codes and exponents staged in
LDS, decoded at the fragment read), several turns of the weight-load ring,
both expert chains in one layer, the full decode layer and the full prefill
layer.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import routed_mixture_experts_amd as moe
import routed_mixture_experts_amd._lib as L
from routed_mixture_experts_amd.synth import WORKLOADS, Workload, make_inputs, random_logits
from tests.helpers import (ExpertFetchMXFP4, WEIGHT_ATOL, check_float, full_layer_parity,
                           lib_cfg, log, np64, npi, oracle_cfg, parity_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mx(inp, **act):
    return moe.ExpertWeights.mxfp4(inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"],
                                   **act)


def _dequant(inp):
    return (O.dequantize_mxfp4(inp["w13"].cpu().numpy(), inp["w13_scale"].cpu().numpy()),
            O.dequantize_mxfp4(inp["w2"].cpu().numpy(), inp["w2_scale"].cpu().numpy()))


@pytest.mark.parametrize("T,E,k,D,I", [
    (50, 16, 2, 256, 256),     # ~6 rows per expert: one 16-row token block
    (200, 8, 2, 384, 256),     # ~50 rows: 2 and 4 token blocks; chunks past K
    (300, 16, 2, 1024, 512),   # ~37 rows, K = 1024: several turns of the load ring
    (700, 8, 3, 384, 256),     # ~260 rows: 256-row tiles with a ragged last tile
    (257, 4, 2, 128, 128),     # N smaller than a tile
    # K a multiple of 1024: workgroups stream 4 column tiles back to back
    (120, 16, 2, 2048, 1024),  # ~15 rows: packed token rows and 1 block
    (400, 16, 2, 1024, 1024),  # ~50 rows: 2 and 4 token blocks
])
def test_experts_mxfp4_match_oracle(T, E, k, D, I):
    log(f"experts mxfp4 T={T} E={E} k={k} D={D} I={I}")
    w = Workload("t", T=T, H=D, E=E, k=k, I=I, weights="mxfp4")
    inp = make_inputs(w, DEV)
    assert inp["w13"].shape == (E, 2 * I, D // 2) and inp["w13_scale"].dtype == torch.uint8
    logits = random_logits(T, E, seed=T + 3).numpy()
    ids, _, _ = O.route(logits, O.RouteCfg(num_experts=E, top_k=k))
    c, off, r2p, p2r = moe.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    y = moe.moe_experts_ex(inp["x"], off, r2p, _mx(inp), k)
    torch.cuda.synchronize()
    _, roff, rr2p, _ = O.permute(ids, E)
    w13, w2 = _dequant(inp)
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, w13, w2)
    log(f"  rows per expert: max {int(np.diff(roff).max())} min {int(np.diff(roff).min())}")
    check_float(np64(y), ref, True, f"y_rows mxfp4 T={T}")


def test_experts_mxfp4_with_activation():
    T, E, k, D, I = 120, 8, 2, 256, 256
    w = Workload("t", T=T, H=D, E=E, k=k, I=I, weights="mxfp4")
    inp = make_inputs(w, DEV)
    ids = np.stack([np.arange(T) % E, (np.arange(T) * 5 + 2) % E], 1)
    c, off, r2p, p2r = moe.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    act = dict(kind="swiglu_clip", alpha=1.702, limit=0.5)
    y = moe.moe_experts_ex(inp["x"], off, r2p,
                           _mx(inp, activation="swiglu_clip", alpha=1.702, limit=0.5), k)
    torch.cuda.synchronize()
    _, roff, rr2p, _ = O.permute(ids, E)
    w13, w2 = _dequant(inp)
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, w13, w2, act)
    check_float(np64(y), ref, True, "y_rows mxfp4 swiglu_clip")


def test_experts_mxfp4_errors():
    lib = moe.load()
    T, E, k, I = 16, 4, 2, 128
    off = torch.zeros((E + 1,), dtype=torch.int32, device=DEV)
    r2p = torch.zeros((T * k,), dtype=torch.int32, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)

    def call(dtype, D, with_scales=True):
        # every case is rejected before any launch
        x = torch.zeros((T, D), dtype=torch.float32 if dtype == L.MOE_DTYPE_F32
                        else torch.bfloat16, device=DEV)
        y = torch.empty((T * k, D), dtype=torch.float32, device=DEV)
        c13 = torch.zeros((E, 2 * I, D // 2), dtype=torch.uint8, device=DEV)
        c2 = torch.zeros((E, D, I // 2), dtype=torch.uint8, device=DEV)
        s13 = torch.full((E, 2 * I, D // 32), 127, dtype=torch.uint8, device=DEV)
        s2 = torch.full((E, D, I // 32), 127, dtype=torch.uint8, device=DEV)
        desc = L.moe_expert_weights_t(L.MOE_WEIGHT_MXFP4, c13.data_ptr(), c2.data_ptr(),
                                      s13.data_ptr() if with_scales else None, s2.data_ptr())
        return lib.moe_experts_ex(dtype, T, k, E, D, I, x.data_ptr(), off.data_ptr(),
                                  r2p.data_ptr(), ctypes.byref(desc), y.data_ptr(),
                                  ws.data_ptr(), ws.numel(), None)

    assert call(L.MOE_DTYPE_F32, 128) == L.MOE_ENOTSUP    # MXFP4 needs a bf16 layer
    assert call(L.MOE_DTYPE_BF16, 192) == L.MOE_ENOTSUP   # D not a multiple of 128
    assert call(L.MOE_DTYPE_BF16, 128, with_scales=False) == L.MOE_EINVAL
    torch.cuda.synchronize()


def test_forward_mxfp4_given_logits_matches_oracle():
    w = Workload("t", T=96, H=256, E=16, k=4, I=128, routed_scaling=2.5, weights="mxfp4")
    log("forward mxfp4 (logits given)")
    inp = make_inputs(w, DEV)
    logits = random_logits(w.T, w.E, seed=6).to(DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    out = moe.moe_forward_ex(lib_cfg(w), inp["x"], _mx(inp), router_logits=logits,
                             topk_ids_out=ids, topk_weights_out=wts)
    torch.cuda.synchronize()
    w13, w2 = _dequant(inp)
    ref = O.forward(np64(inp["x"]), oracle_cfg(w), w13, w2, logits=np64(logits))
    assert (npi(ids) == ref["ids"]).all()
    assert np.abs(np64(wts) - ref["weights"]).max() <= WEIGHT_ATOL
    check_float(np64(out), ref["out"], True, "out mxfp4 small layer")


def test_full_decode_mxfp4():
    """The full decode layer: routing, counts and maps over all 128 tokens
    from the GPU's logits, and the output on 64 tokens against the oracle's
    decode of the same codes."""
    w = WORKLOADS["decode_mxfp4"]
    log(f"full workload decode_mxfp4: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = make_inputs(w, DEV, chunk_rows=16)
    T = w.T
    res = dict(logits=torch.empty((T, w.E), dtype=torch.float32, device=DEV),
               ids=torch.empty((T, w.k), dtype=torch.int32, device=DEV),
               weights=torch.empty((T, w.k), dtype=torch.float32, device=DEV),
               counts=torch.empty((w.E,), dtype=torch.int32, device=DEV))
    res["out"] = moe.moe_forward_ex(lib_cfg(w), inp["x"], _mx(inp), w_router=inp["w_router"],
                                    logits_out=res["logits"], topk_ids_out=res["ids"],
                                    topk_weights_out=res["weights"],
                                    expert_counts_out=res["counts"])
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(1).choice(T, size=64, replace=False))
    full_layer_parity(w, inp, res, ExpertFetchMXFP4(inp["w13"], inp["w13_scale"]),
                      ExpertFetchMXFP4(inp["w2"], inp["w2_scale"]), toks, "decode_mxfp4")
    del inp, res
    torch.cuda.empty_cache()


def test_forward_mxfp4_both_expert_chains():
    """A skewed batch with groups above 64 rows (256x256 tiles, fp16 expert
    rows stored by that kernel) and small groups (streaming, on the
    second stream) in one layer, against the oracle's decode of the codes."""
    w = Workload("t", T=640, H=256, E=16, k=4, I=256, routed_scaling=1.5, weights="mxfp4")
    log("forward mxfp4, both expert chains")
    inp = make_inputs(w, DEV)
    lg = random_logits(w.T, w.E, seed=23)
    lg[:, :4] += 3.0
    lg[:, 4:] += torch.linspace(-2.5, 0.5, w.E - 4)
    logits = lg.to(DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    counts = torch.empty((w.E,), dtype=torch.int32, device=DEV)
    out = moe.moe_forward_ex(lib_cfg(w), inp["x"], _mx(inp), router_logits=logits,
                             topk_ids_out=ids, expert_counts_out=counts)
    torch.cuda.synchronize()
    c = npi(counts)
    log(f"  counts {sorted(c.tolist())}")
    assert c.max() > 128 and ((c > 0) & (c <= 64)).any()
    w13, w2 = _dequant(inp)
    ref = O.forward(np64(inp["x"]), oracle_cfg(w), w13, w2, logits=np64(logits))
    assert (npi(ids) == ref["ids"]).all()
    check_float(np64(out), ref["out"], True, "out mxfp4 both chains")


def test_full_prefill_mxfp4():
    """The prefill layer (T=8192, Zipf(1.1) load) with MXFP4 expert weights:
    routing, counts and maps over every token, the output on at least 64
    tokens (random, the hottest expert's, tokens ending partly filled
    256-row tiles and 16-row token blocks)."""
    w = WORKLOADS["prefill_mxfp4"]
    log(f"full workload prefill_mxfp4: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = make_inputs(w, DEV, chunk_rows=16)
    T = w.T
    res = dict(logits=torch.empty((T, w.E), dtype=torch.float32, device=DEV),
               ids=torch.empty((T, w.k), dtype=torch.int32, device=DEV),
               weights=torch.empty((T, w.k), dtype=torch.float32, device=DEV),
               counts=torch.empty((w.E,), dtype=torch.int32, device=DEV))
    res["out"] = moe.moe_forward_ex(lib_cfg(w), inp["x"], _mx(inp), w_router=inp["w_router"],
                                    router_bias=inp["router_bias"], logits_out=res["logits"],
                                    topk_ids_out=res["ids"], topk_weights_out=res["weights"],
                                    expert_counts_out=res["counts"])
    torch.cuda.synchronize()

    def toks(counts, offsets, r2p):
        t = parity_tokens(w, counts, offsets, r2p, big_rows=256, extra_groups=12)
        extra = np.random.default_rng(2).permutation(T)
        i = 0
        while len(t) < 64:
            t = sorted(set(t) | {int(extra[i])})
            i += 1
        return t

    full_layer_parity(w, inp, res, ExpertFetchMXFP4(inp["w13"], inp["w13_scale"]),
                      ExpertFetchMXFP4(inp["w2"], inp["w2_scale"]), toks, "prefill_mxfp4")
    del inp, res
    torch.cuda.empty_cache()
