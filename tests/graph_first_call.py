"""Run as a script by tests/test_gpu_streams.py: the process's first library
call is made inside a graph capture.  The layer takes both expert chains and
a shared expert, so the capture also creates the library's side stream and
events for the capturing stream.  Replays are compared with eager calls made
afterwards; prints "first-call capture ok" on success."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import routed_mixture_experts_amd as moe  # noqa: E402
from routed_mixture_experts_amd.synth import Workload, make_inputs, random_logits  # noqa: E402


def main():
    dev = "cuda"
    w = Workload("t", T=600, H=256, E=8, k=2, I=128, shared_inter=192)
    inp = make_inputs(w, dev)
    lg = random_logits(w.T, w.E, seed=13)
    lg[:, : w.E // 2] += 2.5          # groups above 64 rows and at most 32
    logits = lg.to(dev)
    cfg = moe.RouteConfig(w.E, w.k)
    sh = dict(w13=inp["w13_sh"], w2=inp["w2_sh"])

    def buffers():
        return dict(out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev),
                    topk_ids_out=torch.empty((w.T, w.k), dtype=torch.int32, device=dev),
                    expert_counts_out=torch.empty((w.E,), dtype=torch.int32, device=dev))

    nbytes = moe.moe_forward_workspace(cfg, torch.bfloat16, w.T, w.H, w.I, None, sh)
    ws_g = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    got, ref = buffers(), buffers()
    torch.cuda.synchronize()
    print("capturing the first library call", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(cfg, inp["x"], inp["w13"], inp["w2"], router_logits=logits,
                        shared=sh, workspace=ws_g, **got)
    torch.cuda.synchronize()
    moe.moe_forward(cfg, inp["x"], inp["w13"], inp["w2"], router_logits=logits, shared=sh,
                    workspace=ws_e, **ref)
    torch.cuda.synchronize()
    c = ref["expert_counts_out"].cpu()
    assert c.max() > 64 and c.min() <= 32, c
    for rep in range(3):
        for t in got.values():
            t.zero_()
        ws_g.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in got.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs"
    print("first-call capture ok", flush=True)


if __name__ == "__main__":
    main()
