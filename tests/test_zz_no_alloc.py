"""moe_forward_noalloc (no workspace: the library's fixed device scratch
array) against moe_forward_ex with a workspace on the same inputs, through
the C ABI.  Two calls in a row, the second with fewer tokens, so the second
runs on scratch contents the first left behind; a layer with a shared expert
and both expert chains (run unsplit on the caller's stream here); and the
decode layer at its full size.  The kernels and their order are the same on
both paths, so the outputs must be identical bit for bit."""
import pytest
import torch

import routed_mixture_experts_amd as moe
from routed_mixture_experts_amd.synth import WORKLOADS, Workload, make_inputs, random_logits
from tests.helpers import check_float, lib_cfg, log, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outs(w, T):
    return dict(out=torch.empty((T, w.H), dtype=torch.bfloat16, device=DEV),
                topk_ids_out=torch.empty((T, w.k), dtype=torch.int32, device=DEV),
                topk_weights_out=torch.empty((T, w.k), dtype=torch.float32, device=DEV),
                expert_counts_out=torch.empty((w.E,), dtype=torch.int32, device=DEV))


def _both(w, inp, T, **kw):
    x = inp["x"][:T].contiguous()
    ex = moe.ExpertWeights(inp["w13"], inp["w2"])
    ref, got = _outs(w, T), _outs(w, T)
    moe.moe_forward_ex(lib_cfg(w), x, ex, **kw, **ref)
    torch.cuda.synchronize()
    for t in got.values():
        t.fill_(-7)
    torch.cuda.synchronize()
    moe.moe_forward_noalloc(lib_cfg(w), x, ex, got["out"], **kw,
                            topk_ids_out=got["topk_ids_out"],
                            topk_weights_out=got["topk_weights_out"],
                            expert_counts_out=got["expert_counts_out"])
    torch.cuda.synchronize()
    return ref, got


def _check(ref, got, tag):
    for name in ref:
        assert torch.equal(ref[name], got[name]), f"{tag}: {name} differs"
    check_float(np64(got["out"]), np64(ref["out"]), True, f"{tag} against moe_forward_ex")


@pytest.mark.parametrize("case", ["router", "shared_two_chains"])
def test_noalloc_matches_forward_ex_two_calls(case):
    if case == "router":
        w = Workload("t", T=300, H=512, E=32, k=4, I=256, routed_scaling=2.0)
        inp = make_inputs(w, DEV)
        kw = dict(w_router=inp["w_router"])
    else:
        w = Workload("t", T=600, H=256, E=8, k=2, I=128, shared_inter=192)
        inp = make_inputs(w, DEV)
        lg = random_logits(w.T, w.E, seed=29)
        lg[:, : w.E // 2] += 2.5      # groups above 64 rows and at most 32
        kw = dict(router_logits=lg.to(DEV), shared=dict(w13=inp["w13_sh"], w2=inp["w2_sh"]))
    for T in (w.T, w.T // 3 + 1):
        log(f"noalloc {case} T={T}")
        kwT = dict(kw)
        if "router_logits" in kwT:
            kwT["router_logits"] = kwT["router_logits"][:T].contiguous()
        ref, got = _both(w, inp, T, **kwT)
        _check(ref, got, f"{case} T={T}")


def test_noalloc_decode_layer_full_size():
    w = WORKLOADS["decode"]
    inp = make_inputs(w, DEV, chunk_rows=16)
    for T in (w.T, 37):
        log(f"noalloc decode T={T}")
        ref, got = _both(w, inp, T, w_router=inp["w_router"])
        _check(ref, got, f"decode T={T}")
    del inp
    torch.cuda.empty_cache()
