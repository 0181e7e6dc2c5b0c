"""GPU parity of the gate/up activation variants (GELU, GELU-tanh, clipped
SwiGLU) against the oracle, on every kernel that applies them: the streaming
kernel (small groups), the 256x256 kernel (large groups, bf16, FP8 or MXFP4
weights) and the fp32 layer's kernel."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import routed_mixture_experts_amd as moe
import routed_mixture_experts_amd._lib as L
from routed_mixture_experts_amd.synth import Workload, make_inputs, random_logits
from tests.helpers import check_float, lib_cfg, log, np64, oracle_cfg

pytestmark = pytest.mark.gpu
DEV = "cuda"

ACTS = {
    "gelu": dict(kind="gelu"),
    "gelu_tanh": dict(kind="gelu_tanh"),
    "swiglu_clip": dict(kind="swiglu_clip", alpha=1.702, limit=7.0),
    # a tight limit, so that many gate/up values are clipped
    "swiglu_clip_tight": dict(kind="swiglu_clip", alpha=1.0, limit=0.5),
}


def _ew(inp, act, fmt="dtype"):
    kw = dict(activation=act["kind"], alpha=act.get("alpha", 1.702), limit=act.get("limit", 7.0))
    if fmt == "fp8_e4m3":
        return moe.ExpertWeights.fp8(inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"], **kw)
    if fmt == "mxfp4":
        return moe.ExpertWeights.mxfp4(inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"],
                                       **kw)
    return moe.ExpertWeights(inp["w13"], inp["w2"], **kw)


@pytest.mark.parametrize("act", list(ACTS))
@pytest.mark.parametrize("dtype,T,E,k,fmt", [
    ("bf16", 50, 16, 2, "dtype"),      # small groups: streaming kernel
    ("bf16", 1200, 4, 2, "dtype"),     # ~600 rows per expert: 256x256 kernel
    ("bf16", 700, 8, 3, "fp8_e4m3"),   # FP8 weights, ~260 rows: 256x256 kernel
    ("bf16", 700, 8, 3, "mxfp4"),      # MXFP4 weights, ~260 rows: 256x256 kernel
    ("f32", 300, 8, 2, "dtype"),       # fp32 layer
])
def test_experts_activation_matches_oracle(act, dtype, T, E, k, fmt):
    D, I = 256, 256 if fmt == "mxfp4" else 192
    log(f"activation {act} {dtype} T={T} E={E} weights={fmt}")
    w = Workload("t", T=T, H=D, E=E, k=k, I=I, dtype=dtype, weights=fmt)
    inp = make_inputs(w, DEV)
    logits = random_logits(T, E, seed=T + 7).numpy()
    ids, _, _ = O.route(logits, O.RouteCfg(num_experts=E, top_k=k))
    c, off, r2p, p2r = moe.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    y = moe.moe_experts_ex(inp["x"], off, r2p, _ew(inp, ACTS[act], fmt), k)
    torch.cuda.synchronize()
    _, roff, rr2p, _ = O.permute(ids, E)
    if fmt == "fp8_e4m3":
        w13 = O.dequantize_rows(inp["w13"].cpu().numpy(), inp["w13_scale"].cpu().numpy())
        w2 = O.dequantize_rows(inp["w2"].cpu().numpy(), inp["w2_scale"].cpu().numpy())
    elif fmt == "mxfp4":
        w13 = O.dequantize_mxfp4(inp["w13"].cpu().numpy(), inp["w13_scale"].cpu().numpy())
        w2 = O.dequantize_mxfp4(inp["w2"].cpu().numpy(), inp["w2_scale"].cpu().numpy())
    else:
        w13, w2 = np64(inp["w13"]), np64(inp["w2"])
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, w13, w2, ACTS[act])
    check_float(np64(y), ref, dtype == "bf16", f"y_rows {act} {dtype}")


def test_forward_with_activation_matches_oracle():
    w = Workload("t", T=96, H=256, E=16, k=4, I=128, routed_scaling=2.5)
    inp = make_inputs(w, DEV)
    logits = random_logits(w.T, w.E, seed=4).to(DEV)
    act = ACTS["swiglu_clip"]
    out = moe.moe_forward_ex(lib_cfg(w), inp["x"], _ew(inp, act), router_logits=logits)
    torch.cuda.synchronize()
    ref = O.forward(np64(inp["x"]), oracle_cfg(w), np64(inp["w13"]), np64(inp["w2"]),
                    logits=np64(logits), act=act)
    check_float(np64(out), ref["out"], True, "out swiglu_clip layer")


def test_activation_errors():
    lib = moe.load()
    T, E, k, D, I = 16, 4, 2, 64, 64
    x = torch.zeros((T, D), dtype=torch.bfloat16, device=DEV)
    off = torch.zeros((E + 1,), dtype=torch.int32, device=DEV)
    r2p = torch.zeros((T * k,), dtype=torch.int32, device=DEV)
    y = torch.empty((T * k, D), dtype=torch.float32, device=DEV)
    w13 = torch.zeros((E, 2 * I, D), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((E, D, I), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)

    def call(act, alpha, limit, n=T):
        # the description is checked before anything else; n = 0 then returns
        # without launching, so the accepted cases run no kernel
        desc = L.moe_expert_weights_t(L.MOE_WEIGHT_DTYPE, w13.data_ptr(), w2.data_ptr(),
                                      None, None, act, alpha, limit)
        return lib.moe_experts_ex(L.MOE_DTYPE_BF16, n, k, E, D, I, x.data_ptr(), off.data_ptr(),
                                  r2p.data_ptr(), ctypes.byref(desc), y.data_ptr(),
                                  ws.data_ptr(), ws.numel(), None)

    clip = L.ACTIVATIONS["swiglu_clip"]
    assert call(4, 1.0, 1.0) == L.MOE_EINVAL        # unknown activation code
    assert call(-1, 1.0, 1.0) == L.MOE_EINVAL
    assert call(clip, 0.0, 7.0) == L.MOE_EINVAL     # clip needs alpha > 0
    assert call(clip, 1.702, -1.0) == L.MOE_EINVAL  # and limit > 0
    assert call(clip, 0.0, 7.0, 0) == L.MOE_EINVAL  # rejected even with no tokens
    assert call(clip, 1.702, 7.0, 0) == L.MOE_OK
    assert call(L.ACTIVATIONS["gelu"], 0.0, 0.0, 0) == L.MOE_OK  # alpha/limit unused off clip
    bad = moe.ExpertWeights(w13, w2, activation="swiglu_clip", limit=0.0)
    with pytest.raises(moe.MoeError):
        moe.moe_experts_ex(x, off, r2p, bad, k)
    with pytest.raises(ValueError):
        moe.ExpertWeights(w13, w2, activation="relu")
    torch.cuda.synchronize()
