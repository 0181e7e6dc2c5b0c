"""Streams, host threads and graph capture at the C ABI.

The library keeps one side stream (with its fork / join / shared-done events)
per caller stream.  These tests check the promises the header makes about
that: buffers the binding allocates belong to the stream the layer runs on;
calls on two streams from two host threads give the results of calls from
one thread; one thread can capture a graph while another runs eagerly; and
the first library call of a process can be made inside a capture.  Every
layer here takes both expert chains and a shared expert, so the side stream
is used.
"""
import os
import subprocess
import sys
import threading

import pytest
import torch

import routed_mixture_experts_amd as moe
from routed_mixture_experts_amd.synth import Workload, make_inputs, random_logits
from tests.helpers import lib_cfg, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
HERE = os.path.dirname(os.path.abspath(__file__))

W = Workload("t", T=600, H=256, E=8, k=2, I=128, shared_inter=192)


def _layer():
    inp = make_inputs(W, DEV)
    lg = random_logits(W.T, W.E, seed=17)
    lg[:, : W.E // 2] += 2.5           # groups above 64 rows and at most 32
    inp["logits"] = lg.to(DEV)
    inp["sh"] = dict(w13=inp["w13_sh"], w2=inp["w2_sh"])
    return inp


def _buffers():
    return dict(out=torch.empty((W.T, W.H), dtype=torch.bfloat16, device=DEV),
                topk_ids_out=torch.empty((W.T, W.k), dtype=torch.int32, device=DEV),
                expert_counts_out=torch.empty((W.E,), dtype=torch.int32, device=DEV))


def _run(inp, x, bufs, ws, stream=None):
    moe.moe_forward(lib_cfg(W), x, inp["w13"], inp["w2"], router_logits=inp["logits"],
                    shared=inp["sh"], workspace=ws, stream=stream, **bufs)


def _ws_bytes(inp):
    return moe.moe_forward_workspace(lib_cfg(W), torch.bfloat16, W.T, W.H, W.I, None, inp["sh"])


def _workspace(inp):
    return torch.empty(_ws_bytes(inp), dtype=torch.uint8, device=DEV)


def _reference(inp, xs):
    refs = []
    for x in xs:
        b = _buffers()
        _run(inp, x, b, _workspace(inp))
        refs.append(b)
    torch.cuda.synchronize()
    c = refs[0]["expert_counts_out"].cpu()
    assert c.max() > 64 and c.min() <= 32, c     # both chains run
    return refs


def test_buffers_made_by_the_binding_belong_to_the_layer_stream():
    """moe_forward on a non-current stream with no workspace and no out: the
    binding allocates both on that stream, so allocations and writes on the
    current stream right after the call cannot take their memory while the
    layer still runs."""
    inp = _layer()
    ref = _reference(inp, [inp["x"]])[0]["out"]
    s = torch.cuda.Stream()
    for rep in range(3):
        s.wait_stream(torch.cuda.current_stream())
        out = moe.moe_forward(lib_cfg(W), inp["x"], inp["w13"], inp["w2"],
                              router_logits=inp["logits"], shared=inp["sh"], stream=s)
        # the current stream allocates blocks of the workspace's size and
        # scribbles on them while the layer runs
        junk = [torch.full((_ws_bytes(inp) // 4,), 7.0 + i, device=DEV) for i in range(8)]
        del junk
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"rep {rep}: output differs from the default-stream run"


def test_two_host_threads_on_two_streams_match_one_thread():
    inp = _layer()
    xs = [inp["x"], (inp["x"].float() * -0.5).to(torch.bfloat16)]
    refs = _reference(inp, xs)
    errors = []
    barrier = threading.Barrier(2)

    def worker(i):
        try:
            s = torch.cuda.Stream()
            ws = _workspace(inp)
            bufs = _buffers()
            torch.cuda.synchronize()
            barrier.wait()
            for rep in range(6):
                with torch.cuda.stream(s):
                    for t in bufs.values():
                        t.zero_()
                    _run(inp, xs[i], bufs, ws, stream=s)
                s.synchronize()
                for name, t in bufs.items():
                    if not torch.equal(t, refs[i][name]):
                        errors.append(f"thread {i} rep {rep}: {name} differs")
                        return
        except Exception as e:  # pragma: no cover - reported below
            errors.append(f"thread {i}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a worker thread did not finish"
    assert not errors, errors


def test_capture_on_one_thread_while_another_runs_eagerly():
    """Thread A captures the layer on its stream (thread-local capture mode)
    while thread B runs the same layer eagerly on another stream; B's side
    stream and events are not A's, so B's work neither joins nor breaks A's
    capture.  Both results match one-thread runs."""
    inp = _layer()
    xs = [inp["x"], (inp["x"].float() * 0.75).to(torch.bfloat16)]
    refs = _reference(inp, xs)
    ws_a, ws_b = _workspace(inp), _workspace(inp)
    got_a, got_b = _buffers(), _buffers()
    s_b = torch.cuda.Stream()
    torch.cuda.synchronize()
    started = threading.Event()
    errors = []

    def eager_b():
        # every torch call of this thread goes to its own stream as well
        try:
            started.wait(timeout=60)
            with torch.cuda.stream(s_b):
                for rep in range(8):
                    _run(inp, xs[1], got_b, ws_b, stream=s_b)
                    s_b.synchronize()
                    for name, t in got_b.items():
                        if not torch.equal(t, refs[1][name]):
                            errors.append(f"eager rep {rep}: {name} differs")
                            return
        except Exception as e:  # pragma: no cover
            errors.append(f"eager thread: {e!r}")

    tb = threading.Thread(target=eager_b)
    tb.start()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        started.set()
        for _ in range(3):   # a longer capture, so the eager calls overlap it
            _run(inp, xs[0], got_a, ws_a)
    tb.join(timeout=120)
    assert not tb.is_alive(), "the eager thread did not finish"
    assert not errors, errors
    for rep in range(2):
        for t in got_a.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in got_a.items():
            assert torch.equal(t, refs[0][name]), f"replay {rep}: {name} differs"


def test_first_library_call_inside_a_graph_capture():
    log("subprocess: first library call inside a capture")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "graph_first_call.py")],
                       capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0, r.returncode
    assert "first-call capture ok" in r.stdout
