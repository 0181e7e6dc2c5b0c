"""Routed-MoE layer throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

A step is one moe_forward (router logits -> scoring/top-k -> permute ->
gate/up+SwiGLU -> down -> combine) over one batch of synthetic tokens already
resident in HBM.  The headline workload is the decode-shaped bf16 layer
(T=128, H=7168, 384 experts, top-8, I=2048, routed scaling 2.5); the
prefill-shaped layer (T=8192, Zipf(1.1) expert load) runs on the same weights
and is reported beside it, and both shapes run again with the same weight
draws quantised to FP8 E4M3 (per-row scales) and to MXFP4 (E2M1 codes, one
E8M0 exponent per 32 elements); each is a separate entry, never the headline
value.  Prints ONE JSON line.

The headline time is a pass with no instrumentation between the kernels.
Per-stage times come from a second pass of as many steps, with HIP events
recorded by the library between its kernels on the timed stream
(``stages_ms``; ``layer_with_stage_events`` is that pass's time per step).  The roofline
entry is the dominant kernel (gate/up + SwiGLU): algorithmic bytes = the
touched experts' gate/up weights + the token activations read + h written.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s
METRIC = "MoE layer tokens/s (T=128 decode, T=8192 prefill); % of HBM/MFMA roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill_zipf", "grouped_sqrtsoftplus", "latent_shared",
                             "decode_fp8", "decode_mxfp4", "prefill_fp8", "prefill_mxfp4"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill line")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the decode and prefill lines with FP8 E4M3 expert weights")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the decode line with MXFP4 expert weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=64)
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--dense-expert", action="store_true",
                    help="also time one dense expert (8192 token rows, H=7168, I=2048, bf16) "
                         "through moe_experts: the 256x256 kernels' gate/up and down alone")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run three plain 1 GiB device-to-device copies (a known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def describe(w) -> str:
    s = (f"{w.name} {w.dtype} T={w.T} H={w.H} E={w.E} top-{w.k} I={w.I} score={w.score}"
         f" renormalize={w.renormalize} routed_scaling={w.routed_scaling}")
    if w.num_groups > 1:
        s += f" groups={w.num_groups} topk_group={w.topk_group} group_score={w.group_score}"
    if w.corr_bias:
        s += f" correction_bias=U(-{w.corr_bias},{w.corr_bias})"
    if w.zipf_s:
        s += f" router_bias=Zipf({w.zipf_s})"
    if w.latent:
        s += f" latent={w.latent}"
    if w.shared_inter:
        s += f" shared_I={w.shared_inter}"
    return s


def layer_work(w, counts):
    """Algorithmic bytes and FLOPs of one forward: touched expert weights,
    router (and dense) weights, x in, out out; intermediates excluded."""
    es = 2 if w.dtype == "bf16" else 4
    D = w.D
    touched = int((counts > 0).sum())
    P = w.T * w.k
    if w.weights == "fp8_e4m3":   # one byte per weight plus an fp32 scale per row
        wbytes = touched * (3 * w.I * D + 4 * (2 * w.I + D)) + w.E * w.H * es
    elif w.weights == "mxfp4":    # half a byte per weight plus a byte per 32
        wbytes = touched * (3 * w.I * D // 2 + 3 * w.I * D // 32) + w.E * w.H * es
    else:
        wbytes = touched * 3 * w.I * D * es + w.E * w.H * es
    flops = 2.0 * P * 3 * D * w.I + 2.0 * w.T * w.H * w.E
    if w.latent:
        wbytes += 2 * w.latent * w.H * es
        flops += 2.0 * w.T * w.H * w.latent * 2
    if w.shared_inter:
        wbytes += 3 * w.shared_inter * w.H * es
        flops += 2.0 * w.T * 3 * w.H * w.shared_inter
    abytes = 2 * w.T * w.H * es
    return wbytes + abytes, flops, touched


# The files the decode gate/up kernel (gemm_bf16_stream) is built from; the
# committed counter summary applies while their hash matches.
STREAM_KERNEL_SOURCES = ("gemm_stream.hip", "gemm_tiles.h", "common.h")

# The decode gate/up + SwiGLU kernel for each expert weight format
# (template arguments: epilogue, K-concatenated, weight format, whole-line
# load pairs, waves per workgroup, column tiles per workgroup).
STREAM_GATE_UP = {"dtype": "gemm_bf16_stream<3, false, 0, true, 8, 1>",
                  "fp8_e4m3": "gemm_bf16_stream<3, false, 1, true, 8, 1>",
                  "mxfp4": "gemm_bf16_stream<3, false, 2, true, 8, 1>"}


def profiled_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when the kernel source no longer
    matches the one the counters were taken on."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "routed_mixture_experts_amd", "csrc")
    h = hashlib.sha256()
    for name in STREAM_KERNEL_SOURCES:
        h.update(open(os.path.join(csrc, name), "rb").read())
    sha = h.hexdigest()[:16]
    for path in glob.glob(os.path.join(ROOT, "profiles", "*hbm_counters*.md")):
        for line in open(path):
            if not line.startswith("traffic:"):
                continue
            kv = dict(f.split("=", 1) for f in line.split()[1:])
            if kv.get("workload") == workload and kv.get("stream_src_sha256_16") == sha:
                return int(kv["bytes_per_launch"])
    return None


def binding_frac(nbytes, flops, ms):
    """Fraction of the binding roofline: max(t_HBM, t_MFMA) / t at the chip's
    peaks (8 TB/s, 2.5 PFLOP/s bf16)."""
    return max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) / (ms * 1e-3)


SEEDS = {"x": 0, "w_router": 1, "w13": 2, "w2": 3, "router_bias": 4, "corr_bias": 5,
         "w_down": 6, "w_up": 7, "w13_sh": 8, "w2_sh": 9, "x_cal": 10, "rank_perm": 11}


def checksums(inp, torch):
    """Sum of every input tensor in float64 (bf16 / fp32 values; FP8 and MXFP4
    weights as their integer codes), taken in slabs: a fingerprint of the
    seeded inputs, outside the timed region."""
    out = {}
    for name, t in inp.items():
        if t is None or not hasattr(t, "dtype"):
            continue
        flat = t.reshape(-1)
        acc = 0.0
        step = 1 << 28
        for i in range(0, flat.numel(), step):
            acc += float(flat[i:i + step].to(torch.float64).sum())
        out[name] = acc
    return out


def gemm1_bytes(w, counts):
    """Algorithmic bytes of one gate/up + SwiGLU launch: gate/up weights of the
    touched experts (unit: one expert, 2*I*D elements), the token activations
    read once, and h written."""
    es = 2 if w.dtype == "bf16" else 4
    touched = int((counts > 0).sum())
    if w.weights == "fp8_e4m3":
        wb = touched * (2 * w.I * w.D + 4 * 2 * w.I)
    elif w.weights == "mxfp4":
        wb = touched * (2 * w.I * w.D // 2 + 2 * w.I * w.D // 32)
    else:
        wb = touched * 2 * w.I * w.D * es
    return wb + w.T * w.D * es + w.T * w.k * w.I * es, touched


def percentile(sorted_vals, q):
    """Linear-interpolated q-th percentile of an ascending list."""
    if len(sorted_vals) == 1:
        return sorted_vals[0]
    pos = (len(sorted_vals) - 1) * q / 100.0
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(sorted_vals) - 1)
    return sorted_vals[lo] + (sorted_vals[hi] - sorted_vals[lo]) * (pos - lo)


class Runner:
    """Holds inputs, outputs, workspace and events of one workload."""

    def __init__(self, w, inp, torch, moe, stream):
        self.w, self.inp, self.torch, self.moe, self.stream = w, inp, torch, moe, stream
        dev = inp["x"].device
        self.cfg = moe.RouteConfig(w.E, w.k, w.num_groups, w.topk_group, w.score,
                                   w.group_score, w.renormalize, w.routed_scaling)
        self.lat = (dict(w_down=inp["w_down"], gamma=inp["gamma"], w_up=inp["w_up"],
                         eps=w.rms_eps) if w.latent else None)
        self.sh = dict(w13=inp["w13_sh"], w2=inp["w2_sh"]) if w.shared_inter else None
        nbytes = moe.moe_forward_workspace(self.cfg, inp["x"].dtype, w.T, w.H, w.I,
                                           self.lat, self.sh)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((w.T, w.H), dtype=inp["x"].dtype, device=dev)
        self.counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
        self.experts = None
        if w.weights == "fp8_e4m3":
            self.experts = moe.ExpertWeights.fp8(inp["w13"], inp["w2"], inp["w13_scale"],
                                                 inp["w2_scale"])
        elif w.weights == "mxfp4":
            self.experts = moe.ExpertWeights.mxfp4(inp["w13"], inp["w2"], inp["w13_scale"],
                                                   inp["w2_scale"])

    def step(self, events=None):
        i = self.inp
        kw = dict(w_router=i["w_router"], router_bias=i["router_bias"],
                  correction_bias=i["corr_bias"], latent=self.lat, shared=self.sh,
                  out=self.out, expert_counts_out=self.counts, stage_events=events,
                  workspace=self.ws, stream=self.stream)
        if self.experts is not None:
            self.moe.moe_forward_ex(self.cfg, i["x"], self.experts, **kw)
        else:
            self.moe.moe_forward(self.cfg, i["x"], i["w13"], i["w2"], **kw)

    def timed(self, steps, warmup):
        torch, moe = self.torch, self.moe
        for _ in range(warmup):
            self.step()
        nev = 2 * moe.MOE_NUM_STAGES
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        for row in evs:             # materialise the HIP events on this stream
            for e in row:
                e.record(self.stream)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        # The headline pass runs the layer as a caller does, with no stage
        # events between its kernels; one event between consecutive steps
        # gives the per-step times (their median, p10 and p90).
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for e in marks:
            e.record(self.stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(self.stream)
        marks[0].record(self.stream)
        for s in range(steps):
            self.step()
            marks[s + 1].record(self.stream)
        end.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(end) / steps
        per_step = sorted(marks[s].elapsed_time(marks[s + 1]) for s in range(steps))
        # A second pass of as many steps records the library's HIP events
        # between the stages, on the stream its kernels run on.
        start.record(self.stream)
        for s in range(steps):
            self.step(evs[s])
        end.record(self.stream)
        torch.cuda.synchronize()
        ms_ev = start.elapsed_time(end) / steps
        stage = {}
        for i, name in enumerate(moe.STAGES):
            d = [evs[s][2 * i].elapsed_time(evs[s][2 * i + 1]) for s in range(steps)]
            stage[name] = sum(d) / steps
        stage["layer_with_stage_events"] = ms_ev
        self.step_stats = {"median": percentile(per_step, 50), "p10": percentile(per_step, 10),
                           "p90": percentile(per_step, 90), "min": per_step[0],
                           "max": per_step[-1]}
        return ms, wall * 1e3 / steps, stage


def cpu_baseline(w, inp, torch, ntok, runs=3):
    """The oracle as it stands, timed on the host cores on the first ``ntok``
    tokens of the batch (routing from its own float64 router product, stable
    permute, per-expert float64 MLPs of the experts those tokens touch,
    combine), ``runs`` times; the median is reported.  Weight copies to the
    host are made before the clock starts."""
    import numpy as np
    import threadpoolctl

    import oracle as O
    x = inp["x"][:ntok].to(torch.float64).cpu().numpy()
    wr = inp["w_router"].to(torch.float64).cpu().numpy()
    rb = None if inp["router_bias"] is None else inp["router_bias"].double().cpu().numpy()
    cb = None if inp["corr_bias"] is None else inp["corr_bias"].double().cpu().numpy()
    cfg = O.RouteCfg(num_experts=w.E, top_k=w.k, num_groups=w.num_groups,
                     topk_group=w.topk_group, score=w.score, group_score=w.group_score,
                     renormalize=w.renormalize, routed_scaling=w.routed_scaling)
    ids, _, _ = O.route(O.router_logits(x, wr, rb), cfg, cb)
    used = sorted(set(ids.reshape(-1).tolist()))
    # host copies (fp32, exact for bf16) of just the experts the sample touches;
    # FP8 / MXFP4 codes are decoded by the oracle (outside the timed region)
    if w.weights in ("fp8_e4m3", "mxfp4"):
        dq = O.dequantize_rows if w.weights == "fp8_e4m3" else O.dequantize_mxfp4
        w13 = {e: dq(inp["w13"][e].cpu().numpy(), inp["w13_scale"][e].cpu().numpy())
               for e in used}
        w2 = {e: dq(inp["w2"][e].cpu().numpy(), inp["w2_scale"][e].cpu().numpy())
              for e in used}
    else:
        w13 = {e: inp["w13"][e].float().cpu().numpy() for e in used}
        w2 = {e: inp["w2"][e].float().cpu().numpy() for e in used}
    # the latent projections and the shared expert, as fp32 host copies
    lat = sh = None
    if w.latent:
        lat = dict(w_down=inp["w_down"].float().cpu().numpy(),
                   gamma=inp["gamma"].float().cpu().numpy(),
                   w_up=inp["w_up"].float().cpu().numpy(), eps=w.rms_eps)
    if w.shared_inter:
        sh = dict(w13=inp["w13_sh"].float().cpu().numpy(),
                  w2=inp["w2_sh"].float().cpu().numpy())
    info = threadpoolctl.threadpool_info()
    cores = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        O.forward(x, cfg, w13, w2, w_router=wr, router_bias=rb, corr_bias=cb, latent=lat,
                  shared=sh)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"first {ntok} of {w.T} tokens of the {w.name} batch ({len(used)} "
                       f"experts touched), numpy float64 oracle forward incl. its own router "
                       f"product; median of {runs} runs: "
                       + ", ".join(f"{t:.2f}" for t in times) + " s")}


def dense_expert(torch, moe, steps: int, warmup: int) -> dict:
    """One expert holding all 8192 token rows (H=7168, I=2048, bf16, seeded
    N(0,1) tokens and N(0,1/fan_in) weights): moe_experts runs the gate/up +
    SwiGLU product and the down product (fp32 rows) on the 256x256 kernels
    with every tile full.  Reports the pair's time and executed rate."""
    from routed_mixture_experts_amd.synth import normal
    T, D, I = 8192, 7168, 2048
    dev = "cuda:0"
    x = normal((T, D), 1.0, 20, torch.bfloat16, dev)
    w13 = normal((1, 2 * I, D), D ** -0.5, 21, torch.bfloat16, dev)
    w2 = normal((1, D, I), I ** -0.5, 22, torch.bfloat16, dev)
    off = torch.tensor([0, T], dtype=torch.int32, device=dev)
    r2p = torch.arange(T, dtype=torch.int32, device=dev)
    y = torch.empty((T, D), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        moe.moe_experts(x, off, r2p, w13, w2, 1, y_rows=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(steps):
        e0.record()
        moe.moe_experts(x, off, r2p, w13, w2, 1, y_rows=y)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    ms = ts[len(ts) // 2]
    flops = 2.0 * T * 3 * D * I
    return {"workload": f"one dense expert: {T} rows, H={D}, I={I}, bf16, fp32 rows out",
            "ms_median": ms, "steps": steps, "algorithmic_flops": flops,
            "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "kernels": "gemm_bf16_big4<3> (gate/up + SwiGLU), gemm_bf16_big4<0> (down, fp32 rows)"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import routed_mixture_experts_amd as moe
    from routed_mixture_experts_amd.synth import WORKLOADS, make_inputs

    moe.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    w = WORKLOADS[args.workload]
    print(f"[bench] generating inputs for {w.name}", file=sys.stderr, flush=True)
    inp = make_inputs(w, dev, chunk_rows=16)
    run = Runner(w, inp, torch, moe, stream)
    print(f"[bench] timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr,
          flush=True)
    ms, wall_ms, stage = run.timed(args.steps, args.warmup)
    counts = run.counts.cpu().numpy()
    abytes, aflops, touched = layer_work(w, counts)
    g1b, _ = gemm1_bytes(w, counts)
    g1_ms = stage["gemm1"]
    g1_gbs = g1b / (g1_ms * 1e-3) / 1e9
    traffic = profiled_traffic(w.name)
    t_s = ms * 1e-3
    res = {
        "metric": METRIC,
        "value": w.T / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_ms": run.step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": describe(w), "tokens": w.T, "touched_experts": touched,
                   "parallelism": "none (1 GPU holds all experts)"},
        "roofline": {"bound": "hbm", "achieved": g1_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": g1_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": (f"gate/up + SwiGLU stage: {STREAM_GATE_UP[w.weights]} (at "
                                "128 tokens every expert's rows, in 64-row tiles)" if w.T <= 128 else
                                "gate/up + SwiGLU stage (both expert chains)"),
                     "kernel_ms": g1_ms, "algorithmic_bytes": g1b},
        "layer": {"hbm_GBps": abytes / t_s / 1e9, "hbm_frac": abytes / t_s / 1e9 / HBM_PEAK_GBS,
                  "mfma_frac": aflops / t_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                  "binding_frac": binding_frac(abytes, aflops, ms),
                  "algorithmic_bytes": abytes, "algorithmic_flops": aflops,
                  "host_wall_ms_per_step": wall_ms},
        "stages_ms": stage,
        "inputs": {"seeds": SEEDS, "checksums": checksums(inp, torch)},
    }
    if args.workload == "decode" and not args.no_prefill:
        wp = WORKLOADS["prefill_zipf"]
        print("[bench] prefill on the same weights", file=sys.stderr, flush=True)
        from routed_mixture_experts_amd.synth import SEED_X, normal, zipf_router_bias
        pin = dict(inp)
        pin["x"] = normal((wp.T, wp.H), 1.0, SEED_X, torch.bfloat16, dev)
        pin["router_bias"] = zipf_router_bias(wp.E, wp.k, wp.T, wp.zipf_s).to(dev)
        prun = Runner(wp, pin, torch, moe, stream)
        psteps = max(3, args.steps // 2)
        pms, _, pstage = prun.timed(psteps, max(1, args.warmup // 2))
        pc = prun.counts.cpu().numpy()
        pbytes, pflops, ptouched = layer_work(wp, pc)
        res["prefill"] = {
            "workload": describe(wp), "value": wp.T / (pms * 1e-3), "unit": "tokens/s",
            "ms_per_step": pms, "step_ms": prun.step_stats, "steps": psteps,
            "hbm_frac": pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": pflops / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "binding_frac": binding_frac(pbytes, pflops, pms),
            "algorithmic_bytes": pbytes, "algorithmic_flops": pflops,
            "load": {"max": int(pc.max()), "min": int(pc.min()), "empty": int((pc == 0).sum()),
                     "histogram": [int(v) for v in pc]},
            "input_checksums": {"x": checksums({"x": pin["x"]}, torch)["x"],
                                "router_bias": checksums({"b": pin["router_bias"]}, torch)["b"]},
            "stages_ms": pstage}
        del prun
    if args.workload == "decode" and not args.no_fp8:
        # the same layer with the same weight draws quantised to FP8 E4M3 (one
        # fp32 scale per weight row): a separate line, not the headline value
        wf = WORKLOADS["decode_fp8"]
        print("[bench] decode with FP8 expert weights", file=sys.stderr, flush=True)
        from routed_mixture_experts_amd.synth import fp8_rows
        fin = dict(inp)
        fin["w13"], fin["w13_scale"] = fp8_rows(inp["w13"])
        fin["w2"], fin["w2_scale"] = fp8_rows(inp["w2"])
        frun = Runner(wf, fin, torch, moe, stream)
        fms, _, fstage = frun.timed(args.steps, args.warmup)
        fc = frun.counts.cpu().numpy()
        fbytes, _, _ = layer_work(wf, fc)
        f1b, _ = gemm1_bytes(wf, fc)
        f1 = f1b / (fstage["gemm1"] * 1e-3) / 1e9
        res["fp8_decode"] = {
            "workload": describe(wf) + " weights=fp8_e4m3 (per-row fp32 scales)",
            "value": wf.T / (fms * 1e-3), "unit": "tokens/s", "ms_per_step": fms,
            "step_ms": frun.step_stats,
            "steps": args.steps, "hbm_frac": fbytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gemm1": {"kernel": STREAM_GATE_UP["fp8_e4m3"], "kernel_ms": fstage["gemm1"],
                      "algorithmic_bytes": f1b, "achieved_GBps": f1, "frac": f1 / HBM_PEAK_GBS,
                      "traffic": profiled_traffic(wf.name)},
            "stages_ms": fstage}
        del frun
        if not args.no_prefill:
            # the prefill batch (same x and router bias row) on the FP8 weights
            wpf = WORKLOADS["prefill_fp8"]
            print("[bench] prefill with FP8 expert weights", file=sys.stderr, flush=True)
            fpin = dict(fin)
            fpin["x"], fpin["router_bias"] = pin["x"], pin["router_bias"]
            fprun = Runner(wpf, fpin, torch, moe, stream)
            fpsteps = max(3, args.steps // 2)
            fpms, _, fpstage = fprun.timed(fpsteps, max(1, args.warmup // 2))
            fpc = fprun.counts.cpu().numpy()
            fpbytes, fpflops, _ = layer_work(wpf, fpc)
            res["fp8_prefill"] = {
                "workload": describe(wpf) + " weights=fp8_e4m3 (per-row fp32 scales)",
                "value": wpf.T / (fpms * 1e-3), "unit": "tokens/s", "ms_per_step": fpms,
                "step_ms": fprun.step_stats, "steps": fpsteps,
                "hbm_frac": fpbytes / (fpms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "mfma_frac": fpflops / (fpms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "binding_frac": binding_frac(fpbytes, fpflops, fpms),
                "algorithmic_bytes": fpbytes, "algorithmic_flops": fpflops,
                "stages_ms": fpstage}
            del fprun, fpin
        del fin
    if args.workload == "decode" and not args.no_mxfp4:
        # the same layer with the same weight draws quantised to MXFP4 (E2M1
        # codes, one E8M0 exponent per 32 elements of a row)
        wm = WORKLOADS["decode_mxfp4"]
        print("[bench] decode with MXFP4 expert weights", file=sys.stderr, flush=True)
        from routed_mixture_experts_amd.synth import mxfp4_rows
        mxin = dict(inp)
        mxin["w13"], mxin["w13_scale"] = mxfp4_rows(inp["w13"])
        mxin["w2"], mxin["w2_scale"] = mxfp4_rows(inp["w2"])
        mrun = Runner(wm, mxin, torch, moe, stream)
        mms, _, mstage = mrun.timed(args.steps, args.warmup)
        mc = mrun.counts.cpu().numpy()
        mbytes, _, _ = layer_work(wm, mc)
        m1b, _ = gemm1_bytes(wm, mc)
        m1 = m1b / (mstage["gemm1"] * 1e-3) / 1e9
        res["mxfp4_decode"] = {
            "workload": describe(wm) + " weights=mxfp4 (E2M1, E8M0 exponent per 32)",
            "value": wm.T / (mms * 1e-3), "unit": "tokens/s", "ms_per_step": mms,
            "step_ms": mrun.step_stats,
            "steps": args.steps, "hbm_frac": mbytes / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "gemm1": {"kernel": STREAM_GATE_UP["mxfp4"], "kernel_ms": mstage["gemm1"],
                      "algorithmic_bytes": m1b, "achieved_GBps": m1, "frac": m1 / HBM_PEAK_GBS,
                      "traffic": profiled_traffic(wm.name)},
            "stages_ms": mstage}
        del mrun
        if not args.no_prefill:
            # the prefill batch (same x and router bias row) on the MXFP4 weights
            wpm = WORKLOADS["prefill_mxfp4"]
            print("[bench] prefill with MXFP4 expert weights", file=sys.stderr, flush=True)
            mpin = dict(mxin)
            mpin["x"], mpin["router_bias"] = pin["x"], pin["router_bias"]
            mprun = Runner(wpm, mpin, torch, moe, stream)
            mpsteps = max(3, args.steps // 2)
            mpms, _, mpstage = mprun.timed(mpsteps, max(1, args.warmup // 2))
            mpc = mprun.counts.cpu().numpy()
            mpbytes, mpflops, _ = layer_work(wpm, mpc)
            res["mxfp4_prefill"] = {
                "workload": describe(wpm) + " weights=mxfp4 (E2M1, E8M0 exponent per 32)",
                "value": wpm.T / (mpms * 1e-3), "unit": "tokens/s", "ms_per_step": mpms,
                "step_ms": mprun.step_stats, "steps": mpsteps,
                "hbm_frac": mpbytes / (mpms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "mfma_frac": mpflops / (mpms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "binding_frac": binding_frac(mpbytes, mpflops, mpms),
                "algorithmic_bytes": mpbytes, "algorithmic_flops": mpflops,
                "stages_ms": mpstage}
            del mprun, mpin
        del mxin
    if args.workload == "decode" and not args.no_prefill:
        del pin
    if args.dense_expert:
        print("[bench] dense expert", file=sys.stderr, flush=True)
        res["dense_expert"] = dense_expert(torch, moe, max(5, args.steps // 2), 2)
    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inp, torch, args.cpu_sample_tokens, args.cpu_runs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
