"""The whole layer captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

moe_forward allocates nothing, synchronises nothing and records no memset, so
a caller can capture it with preallocated outputs and workspace.  When the
batch is large enough to split the experts into a small-group chain on the
library's second stream, that chain is forked from and joined back into the
captured stream with events, and the capture takes it in.  Each replay is
checked against an eager call on the same inputs, with eager work (buffer
clears, a new input copied in) between replays.
"""
import pytest
import torch

import routed_mixture_experts_amd as moe
from routed_mixture_experts_amd.synth import Workload, make_inputs, normal, random_logits
from tests.helpers import lib_cfg, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _skewed_logits(T, E, seed):
    # experts 0 .. E/2-1 get most tokens (groups above 64 rows), the others
    # at most 32: both expert chains run, and the second stream is used
    lg = random_logits(T, E, seed=seed)
    lg[:, : E // 2] += 2.5
    return lg.to(DEV)


# The shared-expert cases fork the shared products onto the second stream at
# the start of the layer and join them before the combine (plain layer) or
# before the latent tail.
@pytest.mark.parametrize("case", ["one_stream", "two_streams", "shared", "latent_shared"])
def test_forward_graph_replays_match_eager(case):
    if case == "one_stream":
        w = Workload("t", T=64, H=256, E=32, k=4, I=128, routed_scaling=2.5)  # P < 16 E
        logits = random_logits(w.T, w.E, seed=11).to(DEV)
    elif case == "two_streams":
        w = Workload("t", T=600, H=256, E=8, k=2, I=128)                     # P >= 16 E
        logits = _skewed_logits(w.T, w.E, seed=12)
    elif case == "shared":
        w = Workload("t", T=600, H=256, E=8, k=2, I=128, shared_inter=192)
        logits = _skewed_logits(w.T, w.E, seed=13)
    else:
        w = Workload("t", T=300, H=512, E=16, k=4, I=128, latent=256, shared_inter=384)
        logits = random_logits(w.T, w.E, seed=14).to(DEV)
    log(f"graph capture {case}: T={w.T} E={w.E} k={w.k}")
    inp = make_inputs(w, DEV)
    cfg = lib_cfg(w)
    lat = None
    if w.latent:
        lat = dict(w_down=inp["w_down"], gamma=inp["gamma"], w_up=inp["w_up"], eps=w.rms_eps)
    sh = dict(w13=inp["w13_sh"], w2=inp["w2_sh"]) if w.shared_inter else None
    x = inp["x"].clone()
    x2 = normal((w.T, w.H), 1.0, 77, torch.bfloat16, DEV)

    def buffers():
        return dict(out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV),
                    topk_ids_out=torch.empty((w.T, w.k), dtype=torch.int32, device=DEV),
                    topk_weights_out=torch.empty((w.T, w.k), dtype=torch.float32, device=DEV),
                    expert_counts_out=torch.empty((w.E,), dtype=torch.int32, device=DEV))

    def run(xin, bufs, ws):
        moe.moe_forward(cfg, xin, inp["w13"], inp["w2"], router_logits=logits, workspace=ws,
                        latent=lat, shared=sh, **bufs)

    nbytes = moe.moe_forward_workspace(cfg, torch.bfloat16, w.T, w.H, w.I, lat, sh)
    ws_e = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws_g = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ref1, ref2 = buffers(), buffers()
    run(x, ref1, ws_e)            # eager (also creates the library's second stream)
    run(x2, ref2, ws_e)
    torch.cuda.synchronize()
    if case in ("two_streams", "shared"):
        c = ref1["expert_counts_out"].cpu()
        assert c.max() > 64 and c.min() <= 32, c   # both chains are exercised

    got = buffers()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(x, got, ws_g)
    torch.cuda.synchronize()
    for rep, (vals, ref) in enumerate([(inp["x"], ref1), (x2, ref2), (inp["x"], ref1),
                                       (x2, ref2)]):
        for t in got.values():
            t.zero_()
        ws_g.fill_(0xA5)           # stale workspace contents must not matter
        x.copy_(vals)              # the captured call reads this buffer
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in got.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs"
