"""GPU parity of moe_experts, moe_combine and moe_forward against the oracle.

Small layers (seconds of oracle time) span several tiles with ragged tails
and are checked element by element; every routing stage there gets the same
logits on both sides, so ids and maps are compared bit for bit.  The full
workloads are run in the configuration the benchmark times: the oracle routes
from the GPU's logits (ids, weights, counts, offsets and maps compared over
every token) and evaluates the output on every token of the small ones and on
at least 64 chosen tokens of the large ones.
"""
import numpy as np
import pytest
import torch

import oracle as O
import routed_mixture_experts_amd as moe
from routed_mixture_experts_amd.synth import WORKLOADS, Workload, make_inputs, random_logits, uniform
from tests.helpers import (WEIGHT_ATOL, ExpertFetch, check_float, check_ids_allowing_near_ties,
                           full_layer_parity, latent_np, lib_cfg, log, np64, npi, oracle_cfg,
                           parity_tokens, shared_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_permute(ids_np, E):
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
    return ids, moe.moe_permute(ids, E)


# ----------------------------------------------------------- experts alone ---

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,E,k,D,I", [
    (50, 16, 2, 256, 192),      # few rows per expert: streaming path for bf16
    (700, 8, 3, 320, 256),      # many rows per expert: tiled path, ragged tiles
    (257, 4, 2, 128, 64),       # N smaller than a tile
    # down product with K = I a multiple of 1024: two column tiles per workgroup
    (120, 16, 2, 512, 1024),    # ~15 rows, some of at most 4 or 8 (packed token loads)
    (200, 16, 2, 256, 2048),    # ~25 rows: 1 and 2 token blocks
])
def test_experts_match_oracle(dtype, T, E, k, D, I):
    log(f"experts {dtype} T={T} E={E} k={k} D={D} I={I}")
    w = Workload("t", T=T, H=D, E=E, k=k, I=I, dtype=dtype)
    inp = make_inputs(w, DEV)
    logits = random_logits(T, E, seed=T).numpy()
    ids, wts, _ = O.route(logits, O.RouteCfg(num_experts=E, top_k=k))
    _, (c, off, r2p, p2r) = _gpu_permute(ids, E)
    y = moe.moe_experts(inp["x"], off, r2p, inp["w13"], inp["w2"], k)
    torch.cuda.synchronize()
    rc, roff, rr2p, rp2r = O.permute(ids, E)
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, np64(inp["w13"]), np64(inp["w2"]))
    check_float(np64(y), ref, dtype == "bf16", f"y_rows {dtype}")


def test_experts_zero_rows_for_most_experts():
    # only 2 of 64 experts get rows; the rest have empty segments
    T, E, k, D, I = 300, 64, 2, 256, 128
    w = Workload("t", T=T, H=D, E=E, k=k, I=I)
    inp = make_inputs(w, DEV)
    ids = np.tile(np.array([5, 40]), (T, 1))
    _, (c, off, r2p, p2r) = _gpu_permute(ids, E)
    y = moe.moe_experts(inp["x"], off, r2p, inp["w13"], inp["w2"], k)
    torch.cuda.synchronize()
    _, roff, rr2p, _ = O.permute(ids, E)
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, np64(inp["w13"]), np64(inp["w2"]))
    check_float(np64(y), ref, True, "y_rows two hot experts")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_combine_matches_oracle(out_dtype):
    T, E, k, D = 333, 24, 6, 512
    g = torch.Generator(device="cpu").manual_seed(2)
    logits = random_logits(T, E, seed=1).numpy()
    ids, wts, _ = O.route(logits, O.RouteCfg(num_experts=E, top_k=k, routed_scaling=1.7))
    _, (c, off, r2p, p2r) = _gpu_permute(ids, E)
    y = torch.randn((T * k, D), generator=g).to(DEV)
    wt = torch.from_numpy(wts.astype(np.float32)).to(DEV)
    out = moe.moe_combine(y, p2r, wt, out_dtype)
    torch.cuda.synchronize()
    _, _, _, rp2r = O.permute(ids, E)
    ref = O.combine(np64(y), rp2r, wts.astype(np.float32).astype(np.float64))
    check_float(np64(out), ref, out_dtype == torch.bfloat16, "combine")


def test_forward_combine_aligned_and_unaligned_out_agree():
    """With fp16 expert rows the combine takes 16-byte row loads and stores
    when its operands are 16-byte aligned, and 8-byte ones otherwise.  Both
    sum the same values in the same order, so a layer output that starts 8
    bytes past a 16-byte boundary is bit-identical to an aligned one."""
    w = Workload("combine_align", T=40, H=512, E=48, k=6, I=256, routed_scaling=2.5)
    inp = make_inputs(w, DEV)
    logits = random_logits(w.T, w.E, seed=41).to(DEV)
    args = (lib_cfg(w), inp["x"], inp["w13"], inp["w2"])
    kw = dict(router_logits=logits, router_bias=inp["router_bias"],
              correction_bias=inp["corr_bias"])
    out_a = moe.moe_forward(*args, **kw)
    big = torch.empty(w.T * w.H + 8, dtype=torch.bfloat16, device=DEV)
    out_u = big[4:4 + w.T * w.H].view(w.T, w.H)
    assert out_a.data_ptr() % 16 == 0 and out_u.data_ptr() % 16 == 8
    moe.moe_forward(*args, out=out_u, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_u)
    ref = _oracle_forward(w, inp, logits=np64(logits))
    check_float(np64(out_u), ref["out"], True, "out, unaligned combine")


# ------------------------------------------------------ whole layer, small ---

SMALL = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "decode_like": Workload("decode_like", T=40, H=512, E=48, k=6, I=256, routed_scaling=2.5),
    # I a multiple of 1024: whole-line weight pairs with no ragged chunk in
    # the streaming down product (all-small batch; two chains)
    "decode_like_i1024": Workload("decode_like_i1024", T=64, H=512, E=32, k=4, I=1024,
                                  routed_scaling=2.5),
    "two_chains_i1024": Workload("two_chains_i1024", T=400, H=512, E=64, k=4, I=1024),
    "prefill_like": Workload("prefill_like", T=600, H=384, E=12, k=4, I=320),
    "grouped_like": Workload("grouped_like", T=300, H=256, E=32, k=4, I=192,
                             score="sqrtsoftplus", num_groups=8, topk_group=4,
                             group_score="top2sum", corr_bias=0.1),
    "latent_like": Workload("latent_like", T=200, H=512, E=16, k=4, I=128, latent=256,
                            shared_inter=192, gamma_std=0.1),
    "latent_noshared": Workload("latent_noshared", T=130, H=256, E=8, k=2, I=128, latent=192),
    # over 256 tokens with K = 1024: the router and the latent down-projection
    # take the K-sliced 128x128 products
    "latent_sliced": Workload("latent_sliced", T=520, H=1024, E=16, k=4, I=128, latent=320,
                              shared_inter=128, gamma_std=0.1),
    "shared_only": Workload("shared_only", T=90, H=256, E=8, k=2, I=128, shared_inter=128),
    "sigmoid_decode": Workload("sigmoid_decode", T=7, H=256, E=64, k=8, I=128,
                               score="sigmoid", renormalize=False, corr_bias=0.2),
    # the largest expert count and top-k the library takes, in a small batch
    # (single-block permute, every group streamed) and a larger one
    "max_experts_topk": Workload("max_experts_topk", T=64, H=256, E=1024, k=32, I=64),
    "max_experts_topk_large": Workload("max_experts_topk_large", T=300, H=256, E=1024, k=32,
                                       I=64, num_groups=16, topk_group=8, score="sigmoid",
                                       group_score="top2sum", corr_bias=0.01),
    "f32_grouped_latent": Workload("f32_grouped_latent", T=70, H=128, E=16, k=4, I=64,
                                   dtype="f32", num_groups=4, topk_group=2, latent=128,
                                   shared_inter=64, gamma_std=0.1),
}


def _oracle_forward(w: Workload, inp: dict, logits=None):
    return O.forward(np64(inp["x"]), oracle_cfg(w), np64(inp["w13"]), np64(inp["w2"]),
                     w_router=np64(inp["w_router"]),
                     router_bias=None if inp["router_bias"] is None else np64(inp["router_bias"]),
                     logits=logits,
                     corr_bias=None if inp["corr_bias"] is None else np64(inp["corr_bias"]),
                     latent=latent_np(inp, w), shared=shared_np(inp, w))


def _gpu_forward(w: Workload, inp: dict, router_logits=None):
    T = inp["x"].shape[0]
    lat = None
    if w.latent:
        lat = dict(w_down=inp["w_down"], gamma=inp["gamma"], w_up=inp["w_up"], eps=w.rms_eps)
    sh = dict(w13=inp["w13_sh"], w2=inp["w2_sh"]) if w.shared_inter else None
    res = dict(
        logits=torch.empty((T, w.E), dtype=torch.float32, device=DEV),
        ids=torch.empty((T, w.k), dtype=torch.int32, device=DEV),
        weights=torch.empty((T, w.k), dtype=torch.float32, device=DEV),
        counts=torch.empty((w.E,), dtype=torch.int32, device=DEV))
    out = moe.moe_forward(lib_cfg(w), inp["x"], inp["w13"], inp["w2"],
                          w_router=None if router_logits is not None else inp["w_router"],
                          router_bias=inp["router_bias"], router_logits=router_logits,
                          correction_bias=inp["corr_bias"], latent=lat, shared=sh,
                          logits_out=res["logits"], topk_ids_out=res["ids"],
                          topk_weights_out=res["weights"], expert_counts_out=res["counts"])
    torch.cuda.synchronize()
    res["out"] = out
    return res


# Router logits of bf16 batches: up to 256 tokens the K-split router
# product; above, 128x128 tiles with K split over slices while their grid is
# under 256 tiles (300..8192 tokens here), else the dense path (257 tokens
# with K = 512 is too short to slice).  Checked against the oracle's float64
# product at the bar of the parity protocol, with and without the bias row,
# for expert counts that do and do not fill whole 16-expert blocks.
@pytest.mark.parametrize("T,H,E", [(1, 256, 16), (17, 512, 1000), (100, 7168, 384),
                                   (128, 7168, 384), (200, 1024, 72), (256, 4096, 256),
                                   (257, 512, 384), (300, 7168, 384), (1000, 1024, 72),
                                   (2048, 7168, 256), (4096, 4096, 256), (8192, 7168, 384)])
@pytest.mark.parametrize("biased", [False, True])
def test_router_logits_small_batches(T, H, E, biased):
    log(f"router logits T={T} H={H} E={E} bias={biased}")
    w = Workload("router", T=T, H=H, E=E, k=2, I=64)
    inp = make_inputs(w, DEV)
    bias = uniform((E,), 2.0, 99, DEV) if biased else None
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    moe.moe_forward(lib_cfg(w), inp["x"], inp["w13"], inp["w2"], w_router=inp["w_router"],
                    router_bias=bias, logits_out=logits)
    torch.cuda.synchronize()
    ref = O.router_logits(np64(inp["x"]), np64(inp["w_router"]),
                          None if bias is None else np64(bias))
    got = np64(logits)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.abs(got - ref).max() / np.sqrt(np.mean(ref * ref))
    log(f"  rel_l2={rel:.2e} max_abs/rms={mx:.2e}")
    assert rel <= 1e-5 and mx <= 1e-4, (rel, mx)


# At most 128 tokens every group is in the streaming list; a group of 65..128
# rows (here: every token on the same k experts) becomes two 64-row tiles.
@pytest.mark.parametrize("T", [65, 100, 128])
def test_forward_hot_experts_small_batch(T):
    w = Workload("hot_small", T=T, H=512, E=16, k=4, I=192, routed_scaling=1.5)
    log(f"forward hot experts T={T}")
    inp = make_inputs(w, DEV)
    logits = random_logits(T, w.E, seed=5)
    logits[:, 3:7] += 20.0   # experts 3..6 win for every token
    logits = logits.to(DEV)
    res = _gpu_forward(w, inp, router_logits=logits)
    ref = _oracle_forward(w, inp, logits=np64(logits))
    assert (npi(res["ids"]) == ref["ids"]).all()
    assert (npi(res["counts"]) == ref["counts"]).all()
    assert sorted(npi(res["counts"])[3:7].tolist()) == [T] * 4
    check_float(np64(res["out"]), ref["out"], True, f"out hot T={T}")


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_given_logits_matches_oracle(name):
    """Same fp32 logits on both sides: routing bit-exact, output in tolerance."""
    w = SMALL[name]
    log(f"forward(logits given) {name}")
    inp = make_inputs(w, DEV)
    logits = random_logits(w.T, w.E, seed=11).to(DEV)
    res = _gpu_forward(w, inp, router_logits=logits)
    ref = _oracle_forward(w, inp, logits=np64(logits))
    assert (npi(res["ids"]) == ref["ids"]).all()
    assert (npi(res["counts"]) == ref["counts"]).all()
    assert np.abs(np64(res["weights"]) - ref["weights"]).max() <= WEIGHT_ATOL
    assert (np64(res["logits"]) == np64(logits)).all()
    check_float(np64(res["out"]), ref["out"], w.dtype == "bf16", f"out {name}")


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_with_router_matches_oracle(name):
    """The router product runs on the GPU: logits in fp32 tolerance, routing
    exact except at float near-ties, output in tolerance on exact tokens."""
    w = SMALL[name]
    log(f"forward(router) {name}")
    inp = make_inputs(w, DEV)
    res = _gpu_forward(w, inp)
    ref = _oracle_forward(w, inp)
    lg = np64(res["logits"])
    rel = np.linalg.norm(lg - ref["logits"]) / np.linalg.norm(ref["logits"])
    assert rel <= 1e-5, rel
    same = check_ids_allowing_near_ties(npi(res["ids"]), ref["ids"], ref["keys"], 1e-5)
    assert same.mean() >= 0.99
    check_float(np64(res["out"])[same], ref["out"][same], w.dtype == "bf16", f"out {name}")


def test_forward_workspace_reused_for_smaller_T():
    """One workspace sized for a capacity serves a smaller batch (buffers come
    from capacity, not the runtime token count)."""
    w = SMALL["prefill_like"]
    inp = make_inputs(w, DEV)
    cfg = lib_cfg(w)
    nbytes = moe.moe_forward_workspace(cfg, torch.bfloat16, w.T, w.H, w.I)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ref = _oracle_forward(w, inp)
    for T in (w.T, 17, w.T - 1):
        x = inp["x"][:T].contiguous()
        out = moe.moe_forward(cfg, x, inp["w13"], inp["w2"], w_router=inp["w_router"],
                              workspace=ws)
        torch.cuda.synchronize()
        sub = O.forward(np64(x), oracle_cfg(w), np64(inp["w13"]), np64(inp["w2"]),
                        w_router=np64(inp["w_router"]))
        check_float(np64(out), sub["out"], True, f"reuse T={T}")
    assert ref is not None


def test_forward_is_deterministic():
    w = SMALL["prefill_like"]
    inp = make_inputs(w, DEV)
    a = _gpu_forward(w, inp)["out"].clone()
    for _ in range(3):
        b = _gpu_forward(w, inp)["out"]
        assert torch.equal(a, b)


def test_forward_two_chains_every_tile_shape():
    """A skewed batch large enough for the two-stream split: groups above 32
    rows in 256-row tiles on the caller's stream (one of 33..64 rows with two
    of its 32-row blocks live), groups of at most 32 rows (1 and 2 token
    blocks of 16 rows) in streaming workgroups on the library's stream."""
    w = Workload("t", T=640, H=256, E=16, k=4, I=192, routed_scaling=1.5)
    inp = make_inputs(w, DEV)
    lg = random_logits(w.T, w.E, seed=21)
    # experts 0-3 take most tokens; 4-15 get graded small loads
    lg[:, :4] += 3.0
    lg[:, 4:] += torch.linspace(-2.5, 0.5, w.E - 4)
    logits = lg.to(DEV)
    res = _gpu_forward(w, inp, router_logits=logits)
    ref = _oracle_forward(w, inp, logits=np64(logits))
    counts = npi(res["counts"])
    log(f"  counts {sorted(counts.tolist())}")
    assert w.T * w.k >= 16 * w.E                        # the two-stream split
    assert counts.max() > 64 and ((counts > 32) & (counts <= 64)).any()
    small = counts[(counts > 0) & (counts <= 32)]
    assert (small <= 16).any() and (small > 16).any()
    assert (npi(res["ids"]) == ref["ids"]).all()
    assert (counts == ref["counts"]).all()
    check_float(np64(res["out"]), ref["out"], True, "out two chains")


def test_forward_groups_just_above_the_streaming_limit():
    """Groups of 33..128 rows (one partly filled 256-row tile each) beside
    larger groups and streaming groups (at most 32 rows) in the same layer."""
    w = Workload("t", T=600, H=256, E=16, k=2, I=192)
    inp = make_inputs(w, DEV)
    lg = random_logits(w.T, w.E, seed=31)
    lg[:, 0] += 1.5
    lg[:, 1] += 1.0
    lg[:, 12:] -= 1.2
    logits = lg.to(DEV)
    res = _gpu_forward(w, inp, router_logits=logits)
    ref = _oracle_forward(w, inp, logits=np64(logits))
    counts = npi(res["counts"])
    log(f"  counts {counts.tolist()}")
    assert ((counts > 64) & (counts <= 128)).sum() >= 2 and (counts > 128).sum() >= 2
    assert ((counts > 32) & (counts <= 64)).sum() >= 2
    assert ((counts > 0) & (counts <= 32)).sum() >= 2
    assert (npi(res["ids"]) == ref["ids"]).all()
    check_float(np64(res["out"]), ref["out"], True, "out groups above 32 rows")


def test_experts_group_sizes_at_tile_class_boundaries():
    """Group sizes on the boundaries of the size classes (streaming up to 32
    rows, 256-row tiles above; one and two tiles around 256; an empty group),
    through moe_experts, element by element against the oracle."""
    sizes = [32, 33, 64, 65, 128, 129, 1, 256, 257, 0, 3]
    E, k, D, I = len(sizes), 2, 256, 128
    labels = np.repeat(np.arange(E), sizes)          # sorted expert labels
    T = len(labels) // k
    ids = np.stack([labels[:T], labels[T:]], 1)       # distinct per token
    assert (ids[:, 0] != ids[:, 1]).all()
    w = Workload("t", T=T, H=D, E=E, k=k, I=I)
    inp = make_inputs(w, DEV)
    c, off, r2p, p2r = moe.moe_permute(torch.from_numpy(ids.astype(np.int32)).to(DEV), E)
    assert npi(c).tolist() == sizes
    y = moe.moe_experts(inp["x"], off, r2p, inp["w13"], inp["w2"], k)
    torch.cuda.synchronize()
    _, roff, rr2p, _ = O.permute(ids, E)
    ref = O.run_experts(np64(inp["x"]), k, roff, rr2p, np64(inp["w13"]), np64(inp["w2"]))
    check_float(np64(y), ref, True, "y_rows size-class boundaries")


def test_forward_empty_batch():
    w = SMALL["decode_like"]
    inp = make_inputs(w, DEV)
    x = inp["x"][:0]
    out = moe.moe_forward(lib_cfg(w), x, inp["w13"], inp["w2"], w_router=inp["w_router"])
    torch.cuda.synchronize()
    assert out.shape == (0, w.H)


# ------------------------------------------------------ full workloads ---

FULL = ["tiny_fp32", "decode", "prefill_zipf", "grouped_sqrtsoftplus", "latent_shared"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    """Every workload at its full size, in the launch configuration the
    benchmark times.  Routing, counts, offsets and maps are compared bit for
    bit over all tokens (the oracle routes from the GPU's logits); the output
    element by element on every token of the tiny and decode layers, and on
    at least 64 tokens of the others: random ones, the hottest expert's, and
    tokens whose rows end partly filled tiles."""
    w = WORKLOADS[name]
    log(f"full workload {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I}")
    inp = make_inputs(w, DEV, chunk_rows=16)
    res = _gpu_forward(w, inp)
    if w.T <= 128:
        toks = list(range(w.T))
    else:
        def toks(counts, offsets, r2p):
            t = parity_tokens(w, counts, offsets, r2p)
            extra = np.random.default_rng(1).permutation(w.T)
            i = 0
            while len(t) < 64:
                t = sorted(set(t) | {int(extra[i])})
                i += 1
            return t
    full_layer_parity(w, inp, res, ExpertFetch(inp["w13"]), ExpertFetch(inp["w2"]), toks, name)
    del inp, res
    torch.cuda.empty_cache()
