"""GPU parity of the FP8 E4M3 expert-weight path (moe_experts_ex,
moe_forward_ex) against the oracle.

The oracle decodes the same codes and row scales into float64 weights
(oracle.dequantize_rows), so both sides multiply by exactly the same weight
values; the remaining difference is the bf16 rounding of h and of the output,
and the bar is the bf16 layer's.  Shapes cover the streaming kernel with 1, 2
and 4 token blocks and a ragged last K chunk, the 256x256 kernel (codes
staged in LDS) for groups above 64 rows, both expert chains in one layer, and
the full decode and prefill layers.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import routed_mixture_experts_amd as moe
import routed_mixture_experts_amd._lib as L
from routed_mixture_experts_amd.synth import WORKLOADS, Workload, make_inputs, random_logits
from tests.helpers import (ExpertFetchFP8, WEIGHT_ATOL, check_float, full_layer_parity, lib_cfg,
                           log, np64, npi, oracle_cfg, parity_tokens)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _fp8(inp):
    return moe.ExpertWeights.fp8(inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"])


def _dequant(inp):
    return (O.dequantize_rows(inp["w13"].cpu().numpy(), inp["w13_scale"].cpu().numpy()),
            O.dequantize_rows(inp["w2"].cpu().numpy(), inp["w2_scale"].cpu().numpy()))


@pytest.mark.parametrize("T,E,k,D,I", [
    (50, 16, 2, 256, 192),     # ~6 rows per expert: one 16-row token block
    (200, 8, 2, 320, 256),     # ~50 rows: 2 and 4 token blocks, K = 320 ends mid-chunk
    (700, 8, 3, 320, 256),     # ~260 rows: a full and a ragged 256-row tile
    (257, 4, 2, 128, 64),      # N smaller than a tile
    # K a multiple of 128: whole-line weight load pairs
    (120, 16, 2, 1024, 512),   # ~15 rows: 1 token block
    (320, 16, 2, 512, 256),    # ~40 rows: 2 and 4 token blocks
    # down product with K = I a multiple of 1024: two column tiles per workgroup
    (120, 16, 2, 512, 1024),   # ~15 rows: 1 token block
    (200, 16, 2, 256, 1024),   # ~25 rows: 1 and 2 token blocks
    (320, 16, 2, 256, 2048),   # ~40 rows: 4 token blocks (4 loads in flight)
])
def test_experts_fp8_match_oracle(T, E, k, D, I):
    log(f"experts fp8 T={T} E={E} k={k} D={D} I={I}")
    w = Workload("t", T=T, H=D, E=E, k=k, I=I, weights="fp8_e4m3")
    inp = make_inputs(w, DEV)
    assert inp["w13"].dtype == torch.uint8
    logits = random_logits(T, E, seed=T + 1).numpy()
    ids, _, _ = O.route(logits, O.RouteCfg(num_experts=E, top_k=k))
    c, off, r2p, p2r = moe.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    y = moe.moe_experts_ex(inp["x"], off, r2p, _fp8(inp), k)
    torch.cuda.synchronize()
    _, roff, rr2p, _ = O.permute(ids, E)
    w13, w2 = _dequant(inp)
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, w13, w2)
    log(f"  rows per expert: max {int(np.diff(roff).max())} min {int(np.diff(roff).min())}")
    check_float(np64(y), ref, True, f"y_rows fp8 T={T}")


def test_experts_ex_dtype_format_equals_moe_experts():
    T, E, k, D, I = 300, 8, 2, 256, 128
    w = Workload("t", T=T, H=D, E=E, k=k, I=I)
    inp = make_inputs(w, DEV)
    ids = np.stack([np.arange(T) % E, (np.arange(T) * 3 + 1) % E], 1)
    c, off, r2p, p2r = moe.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    y0 = moe.moe_experts(inp["x"], off, r2p, inp["w13"], inp["w2"], k)
    y1 = moe.moe_experts_ex(inp["x"], off, r2p, moe.ExpertWeights(inp["w13"], inp["w2"]), k)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_experts_ex_errors():
    lib = moe.load()
    T, E, k, D, I = 16, 4, 2, 64, 64
    x = torch.zeros((T, D), dtype=torch.float32, device=DEV)
    off = torch.zeros((E + 1,), dtype=torch.int32, device=DEV)
    r2p = torch.zeros((T * k,), dtype=torch.int32, device=DEV)
    y = torch.empty((T * k, D), dtype=torch.float32, device=DEV)
    codes13 = torch.zeros((E, 2 * I, D), dtype=torch.uint8, device=DEV)
    codes2 = torch.zeros((E, D, I), dtype=torch.uint8, device=DEV)
    s13 = torch.ones((E, 2 * I), dtype=torch.float32, device=DEV)
    s2 = torch.ones((E, D), dtype=torch.float32, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)

    def call(dtype, desc):
        return lib.moe_experts_ex(dtype, T, k, E, D, I, x.data_ptr(), off.data_ptr(),
                                  r2p.data_ptr(), ctypes.byref(desc) if desc else None,
                                  y.data_ptr(), ws.data_ptr(), ws.numel(), None)

    fp8 = L.moe_expert_weights_t(L.MOE_WEIGHT_FP8_E4M3, codes13.data_ptr(), codes2.data_ptr(),
                                 s13.data_ptr(), s2.data_ptr())
    assert call(L.MOE_DTYPE_F32, fp8) == L.MOE_ENOTSUP       # FP8 needs a bf16 layer
    bad = L.moe_expert_weights_t(7, codes13.data_ptr(), codes2.data_ptr(), None, None)
    assert call(L.MOE_DTYPE_BF16, bad) == L.MOE_EINVAL       # unknown format
    assert call(L.MOE_DTYPE_BF16, None) == L.MOE_EINVAL      # no description
    xb = x.to(torch.bfloat16)
    noscale = L.moe_expert_weights_t(L.MOE_WEIGHT_FP8_E4M3, codes13.data_ptr(),
                                     codes2.data_ptr(), None, s2.data_ptr())
    st = lib.moe_experts_ex(L.MOE_DTYPE_BF16, T, k, E, D, I, xb.data_ptr(), off.data_ptr(),
                            r2p.data_ptr(), ctypes.byref(noscale), y.data_ptr(), ws.data_ptr(),
                            ws.numel(), None)
    assert st == L.MOE_EINVAL                                # missing w13 scales
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,H,E,k,I", [
    (96, 256, 16, 4, 128),
    # I a multiple of 1024: the streaming down product's workgroups take two
    # column tiles each (an all-small batch; a batch with both chains)
    (64, 512, 32, 4, 1024),
    (400, 512, 64, 4, 1024),
])
def test_forward_fp8_given_logits_matches_oracle(T, H, E, k, I):
    w = Workload("t", T=T, H=H, E=E, k=k, I=I, routed_scaling=2.5, weights="fp8_e4m3")
    log(f"forward fp8 (logits given) T={T} H={H} E={E} k={k} I={I}")
    inp = make_inputs(w, DEV)
    logits = random_logits(w.T, w.E, seed=5).to(DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    out = moe.moe_forward_ex(lib_cfg(w), inp["x"], _fp8(inp), router_logits=logits,
                             topk_ids_out=ids, topk_weights_out=wts)
    torch.cuda.synchronize()
    w13, w2 = _dequant(inp)
    ref = O.forward(np64(inp["x"]), oracle_cfg(w), w13, w2, logits=np64(logits))
    assert (npi(ids) == ref["ids"]).all()
    assert np.abs(np64(wts) - ref["weights"]).max() <= WEIGHT_ATOL
    check_float(np64(out), ref["out"], True, "out fp8 small layer")


def test_full_decode_fp8():
    """The full decode layer: routing, counts and maps over all 128 tokens
    from the GPU's logits, and the output on 64 tokens against the oracle's
    decode of the same codes."""
    w = WORKLOADS["decode_fp8"]
    log(f"full workload decode_fp8: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = make_inputs(w, DEV, chunk_rows=16)
    T = w.T
    res = dict(logits=torch.empty((T, w.E), dtype=torch.float32, device=DEV),
               ids=torch.empty((T, w.k), dtype=torch.int32, device=DEV),
               weights=torch.empty((T, w.k), dtype=torch.float32, device=DEV),
               counts=torch.empty((w.E,), dtype=torch.int32, device=DEV))
    res["out"] = moe.moe_forward_ex(lib_cfg(w), inp["x"], _fp8(inp), w_router=inp["w_router"],
                                    logits_out=res["logits"], topk_ids_out=res["ids"],
                                    topk_weights_out=res["weights"],
                                    expert_counts_out=res["counts"])
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(0).choice(T, size=64, replace=False))
    full_layer_parity(w, inp, res, ExpertFetchFP8(inp["w13"], inp["w13_scale"]),
                      ExpertFetchFP8(inp["w2"], inp["w2_scale"]), toks, "decode_fp8")
    del inp, res
    torch.cuda.empty_cache()


def test_forward_fp8_both_expert_chains():
    """A skewed batch with groups above 64 rows (256-row tiles, fp16 expert
    rows stored by the 256x256 kernel) and small groups (streaming, on the
    second stream) in one layer, against the oracle's decode of the codes."""
    w = Workload("t", T=640, H=256, E=16, k=4, I=192, routed_scaling=1.5, weights="fp8_e4m3")
    log("forward fp8, both expert chains")
    inp = make_inputs(w, DEV)
    lg = random_logits(w.T, w.E, seed=23)
    lg[:, :4] += 3.0
    lg[:, 4:] += torch.linspace(-2.5, 0.5, w.E - 4)
    logits = lg.to(DEV)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
    counts = torch.empty((w.E,), dtype=torch.int32, device=DEV)
    out = moe.moe_forward_ex(lib_cfg(w), inp["x"], _fp8(inp), router_logits=logits,
                             topk_ids_out=ids, expert_counts_out=counts)
    torch.cuda.synchronize()
    c = npi(counts)
    log(f"  counts {sorted(c.tolist())}")
    assert c.max() > 128 and ((c > 0) & (c <= 64)).any()
    w13, w2 = _dequant(inp)
    ref = O.forward(np64(inp["x"]), oracle_cfg(w), w13, w2, logits=np64(logits))
    assert (npi(ids) == ref["ids"]).all()
    check_float(np64(out), ref["out"], True, "out fp8 both chains")


def test_full_prefill_fp8():
    """The prefill layer (T=8192, Zipf(1.1) load) with FP8 expert weights:
    routing, counts and maps over every token, the output on at least 64
    tokens (random, the hottest expert's, tokens ending partly filled
    256-row tiles and 16-row token blocks)."""
    w = WORKLOADS["prefill_fp8"]
    log(f"full workload prefill_fp8: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = make_inputs(w, DEV, chunk_rows=16)
    T = w.T
    res = dict(logits=torch.empty((T, w.E), dtype=torch.float32, device=DEV),
               ids=torch.empty((T, w.k), dtype=torch.int32, device=DEV),
               weights=torch.empty((T, w.k), dtype=torch.float32, device=DEV),
               counts=torch.empty((w.E,), dtype=torch.int32, device=DEV))
    res["out"] = moe.moe_forward_ex(lib_cfg(w), inp["x"], _fp8(inp), w_router=inp["w_router"],
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

    full_layer_parity(w, inp, res, ExpertFetchFP8(inp["w13"], inp["w13_scale"]),
                      ExpertFetchFP8(inp["w2"], inp["w2_scale"]), toks, "prefill_fp8")
    del inp, res
    torch.cuda.empty_cache()
