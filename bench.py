#!/usr/bin/env python3
"""Throughput of the MI355X selective scan (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mamba130m]

A step is one ssm_scan_fwd call over a whole batch of the workload (discretise,
scan, carry, output epilogue: the entire prefill/training-forward path) with
every input already resident in HBM.  The timed loop rotates through enough
independent input sets that they cannot be served from the 256 MB Infinity
Cache.  The same JSON line also carries the decode path (ssm_state_update) on
the 2.8B-shaped generation workload, the backward pass (ssm_scan_bwd; as context
also its ZOH variant and ssm_scan_bwd_saved from a saving forward's checkpoints) on
the same workload, the conv + SiLU step that produces u
(ssm_conv1d_fwd on the same [B, D, L] shape, ssm_conv1d_update on the decode
shape) and the fp64 CPU oracle's rate on the host.

Progress goes to stderr; stdout gets exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "selective-scan state updates/sec (B·L·D·N) and HBM GB/s % of peak, 1 MI355X"
HBM_PEAK_GBS = 8000.0
# ALU roofline of the scan.  A state update needs, at minimum, 5 fp32 operations: the exp2
# argument (mul), exp2 (v_exp_f32), B_bar*u (mul), the state update (FMA) and C*h (FMA).
# Measured issue cost on gfx950 with >= 2 waves per SIMD (two waves issue VALU concurrently):
# 1.9 clk per wave64 plain fp32 op and 5.5 clk per v_exp_f32.  The peak rate of this op mix is
# 5 ops per (4 * 1.9 + 5.5) clk per 64 lanes per SIMD, over 1024 SIMDs at 2.4 GHz.
OPS_PER_UPDATE = 5
ALU_PEAK_TOPS = OPS_PER_UPDATE * 64 / (4 * 1.9 + 5.5) * 1024 * 2.4e9 / 1e12
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    csrc = os.path.join(ROOT, "selective_state_space_76_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def scan_bytes(w) -> int:
    """Algorithmic HBM bytes of one scan call: each input read once, each output written once."""
    s = 4 if w.io == "f32" else 2
    BDL, BNL = w.batch * w.dim * w.seqlen, w.batch * w.dstate * w.seqlen
    return (3 * s * BDL + s * BDL + 2 * s * BNL + 4 * w.dim * w.dstate + 4 * w.dim * (2 if w.bias else 1)
            + 4 * w.batch * w.dim * w.dstate)


def step_bytes(w) -> int:
    """Algorithmic HBM bytes of one decode step: state read + written, per-token streams, params."""
    s = 4 if w.io == "f32" else 2
    BD, BDN = w.batch * w.dim, w.batch * w.dim * w.dstate
    return 2 * 4 * BDN + 4 * s * BD + 2 * s * w.batch * w.dstate + 4 * w.dim * w.dstate + 8 * w.dim


def traffic_from_profile(workload: str, launches_per_call: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the built kernels."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def bench_scan(args, torch, ssm, W):
    w = W.WORKLOADS[args.workload]
    per_set = scan_bytes(w)
    R = max(1, min(8, math.ceil(2 * MALL_BYTES / per_set)))
    log("workload %s %s, %d rotated input sets of %.1f MB" % (w.name, (w.batch, w.dim, w.dstate, w.seqlen),
                                                                R, per_set / 1e6))
    sets = []
    for k in range(R):
        x = W.scan_inputs(w.with_shape(seed=w.seed + 1000 * k), device="cuda")
        x["out"] = torch.empty_like(x["u"])
        x["fs"] = torch.empty(w.batch, w.dim, w.dstate, device="cuda")
        sets.append(x)
    need = ssm.workspace_size(w.batch, w.dim, w.dstate, w.seqlen, ssm.SSM_BF16 if w.io == "bf16" else ssm.SSM_F32)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None

    def call(x):
        ssm.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                     out=x["out"], final_state=x["fs"], workspace=ws)

    for k in range(args.warmup):
        call(sets[k % R])
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record()
        call(sets[k % R])
        ends[k].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    ms_step = (t1 - t0) * 1e3 / args.steps
    mean_launch = sum(launch_ms) / len(launch_ms)
    # the same launch with L2 and the Infinity Cache flushed before each rep (a 1 GiB fill outside
    # the events), as a cross-check of the rotation above
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    nf = min(args.steps, 20)
    fs_, fe_ = [torch.cuda.Event(enable_timing=True) for _ in range(nf)], [torch.cuda.Event(enable_timing=True) for _ in range(nf)]
    for k in range(nf):
        flush.zero_()
        fs_[k].record()
        call(sets[k % R])
        fe_[k].record()
    torch.cuda.synchronize()
    flushed = sorted(s_.elapsed_time(e_) for s_, e_ in zip(fs_, fe_))
    del flush
    return w, R, ms_step, mean_launch, launch_ms, sets[0], flushed


def bench_decode(args, torch, ssm, W):
    w = W.WORKLOADS["decode2p8b"]
    steps = args.decode_steps
    A, Dv, bias = W.params(w, device="cuda")
    nstate = max(1, math.ceil(1.25 * MALL_BYTES / (4 * w.batch * w.dim * w.dstate)))
    states = [torch.zeros(w.batch, w.dim, w.dstate, device="cuda") for _ in range(nstate)]
    log("decode %s x %d steps, %d rotated state buffers" % ((w.batch, w.dim, w.dstate), steps, nstate))
    inputs = [W.decode_inputs(w, k, device="cuda") for k in range(steps)]
    outs = [torch.empty(w.batch, w.dim, dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def step(k):
        x = inputs[k]
        ssm.state_update(states[k % nstate], x["u"], x["delta"], A, x["B"], x["C"], Dv, x["z"], bias,
                         out=outs[k % 2])

    for k in range(min(20, steps)):
        step(k)
    for s in states:
        s.zero_()
    torch.cuda.synchronize()
    # one event per 50 steps: an event between every pair of steps would add its own gap to the queue
    chunk = 50 if steps >= 100 else 1
    marks = list(range(0, steps + 1, chunk))
    if marks[-1] != steps:
        marks.append(steps)
    ev = {m: torch.cuda.Event(enable_timing=True) for m in marks}
    t0 = time.perf_counter()
    ev[0].record()
    for k in range(steps):
        step(k)
        if k + 1 in ev:
            ev[k + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = sorted(ev[a].elapsed_time(ev[b]) / (b - a) for a, b in zip(marks[:-1], marks[1:]))
    ms_step = (t1 - t0) * 1e3 / steps
    eager_gpu_ms = ev[0].elapsed_time(ev[steps]) / steps
    # The eager loop can be bound by the Python binding's per-call cost; the same steps captured once
    # in a HIP graph and replayed back to back measure the device (how a serving loop issues them).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for k in range(steps):
            step(k)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    gpu_ms = g0.elapsed_time(g1) / steps
    del graph
    # the same steps on a single state buffer (84 MB, resident in the 256 MB Infinity Cache): the
    # cache-warm rate, for comparison only
    warm = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(warm, stream=side):
        for k in range(steps):
            x = inputs[k]
            ssm.state_update(states[0], x["u"], x["delta"], A, x["B"], x["C"], Dv, x["z"], bias, out=outs[k % 2])
    torch.cuda.current_stream().wait_stream(side)
    warm.replay()
    torch.cuda.synchronize()
    g0.record()
    warm.replay()
    g1.record()
    torch.cuda.synchronize()
    warm_ms = g0.elapsed_time(g1) / steps
    del warm
    upd = w.batch * w.dim * w.dstate
    b = step_bytes(w)
    return {
        "workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "steps": steps,
        "rotated_state_buffers": nstate,
        "value": upd / (gpu_ms * 1e-3), "unit": "state-updates/s", "eager_wall_ms_per_step": ms_step,
        "gpu_ms_per_step": gpu_ms, "timing": "HIP graph of the steps, replayed",
        "mall_warm_gpu_ms_per_step": warm_ms,
        "eager_gpu_ms_per_step": eager_gpu_ms, "eager_median_step_ms": per[len(per) // 2],
        "eager_step_ms_from": "events every %d steps" % chunk,
        "roofline": {"bound": "hbm", "achieved": b / (gpu_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": b / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic_from_profile(w.name, 1),
                     "algorithmic_bytes_per_step": b},
    }


def bwd_bytes(w) -> int:
    """Algorithmic HBM bytes of one backward call: the forward's inputs and dout read once,
    du, ddelta and dz written once, dB, dC (fp32) and the per-channel gradients written once."""
    s = 4 if w.io == "f32" else 2
    BDL, BNL = w.batch * w.dim * w.seqlen, w.batch * w.dstate * w.seqlen
    return (4 * s * BDL + 2 * s * BNL + 3 * s * BDL + 2 * 4 * BNL + 2 * 4 * w.dim * w.dstate
            + 4 * 4 * w.dim)


def bench_bwd(args, torch, ssm, W):
    """One ssm_scan_bwd call per step on the scan workload (checkpoint pass, backward pass and
    the fixed-order partial sums), inputs rotated past the Infinity Cache."""
    w = W.WORKLOADS[args.workload]
    per_set = bwd_bytes(w)
    R = max(1, min(4, math.ceil(2 * MALL_BYTES / per_set)))
    sets = []
    for k in range(R):
        x = W.scan_inputs(w.with_shape(seed=w.seed + 1000 * k), device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed + 77 + k)
        x["dout"] = torch.randn(w.batch, w.dim, w.seqlen, generator=g, device="cuda").to(x["u"].dtype)
        sets.append(x)
    need = ssm.bwd_workspace_size(w.batch, w.dim, w.dstate, w.seqlen,
                                  ssm.SSM_BF16 if w.io == "bf16" else ssm.SSM_F32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    grads = None

    def call(x, zoh=False, saved=False):
        nonlocal grads
        grads = ssm.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                             dout=x["dout"], grads=grads, workspace=ws, zoh=zoh,
                             checkpoints=x["ck"] if saved else None)

    def timed(n, zoh, saved=False):
        for k in range(max(2, args.warmup)):
            call(sets[k % R], zoh, saved)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        torch.cuda.synchronize()
        for k in range(n):
            ev[2 * k].record()
            call(sets[k % R], zoh, saved)
            ev[2 * k + 1].record()
        torch.cuda.synchronize()
        return sorted(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(n))

    n = max(5, args.steps // 2)
    ms = timed(n, False)
    mean = sum(ms) / n
    mz = timed(5, True)  # the zero-order-hold variant, same inputs (context, not the bench value)
    # context: the backward from the checkpoints a saving forward wrote (ssm_scan_bwd_saved), as a
    # training step runs it; the forward that wrote them is outside the timed calls
    for x in sets:
        x["ck"] = torch.empty(ssm.checkpoints_shape(w.batch, w.dim, w.dstate, w.seqlen), device="cuda")
        ssm.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                     checkpoints=x["ck"])
    msv = timed(n, False, saved=True)
    b = bwd_bytes(w)
    return {"workload": w.name, "rotated_input_sets": R, "call_ms": mean, "call_ms_median": ms[n // 2],
            "value": w.updates / (mean * 1e-3), "unit": "state-updates/s",
            "workspace_bytes": need, "algorithmic_bytes_per_call": b,
            "hbm_GBs": b / (mean * 1e-3) / 1e9, "zoh_call_ms": sum(mz) / len(mz),
            "from_saved_checkpoints_call_ms": sum(msv) / len(msv)}


def conv_bytes(w, K) -> int:
    """Algorithmic HBM bytes of one conv prefill call: x read, u written, the carried-out state
    written, weights and bias read."""
    s = 4 if w.io == "f32" else 2
    BDL, BD = w.batch * w.dim * w.seqlen, w.batch * w.dim
    return 2 * s * BDL + s * BD * (K - 1) + 4 * w.dim * (K + 1)


def conv_step_bytes(w, K) -> int:
    """Algorithmic HBM bytes of one conv decode step: state read + written, x read, u written,
    weights and bias read."""
    s = 4 if w.io == "f32" else 2
    BD = w.batch * w.dim
    return 2 * s * BD * (K - 1) + 2 * s * BD + 4 * w.dim * (K + 1)


def bench_conv(args, torch, ssm, W, K=4):
    """The conv + SiLU step that produces u, on the scan workload's [B, D, L] shape, and its
    decode form on the generation workload; events bracket each launch on the launch stream."""
    w = W.WORKLOADS[args.workload]
    per_set = conv_bytes(w, K)
    R = max(1, min(8, math.ceil(2 * MALL_BYTES / per_set)))
    sets = []
    for k in range(R):
        c = W.conv_inputs(w.with_shape(seed=w.seed + 1000 * k), K, device="cuda")
        c["u"] = torch.empty_like(c["x"])
        c["so"] = torch.empty((w.batch, w.dim, K - 1), dtype=c["x"].dtype, device="cuda")
        sets.append(c)
    for k in range(args.warmup):
        c = sets[k % R]
        ssm.conv1d_fwd(c["x"], c["weight"], c["bias"], out=c["u"], final_state=c["so"])
    n = max(args.steps, 20)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    torch.cuda.synchronize()
    for k in range(n):
        c = sets[k % R]
        ev[2 * k].record()
        ssm.conv1d_fwd(c["x"], c["weight"], c["bias"], out=c["u"], final_state=c["so"])
        ev[2 * k + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(n))
    mean = sum(ms) / n
    b = conv_bytes(w, K)
    pre = {"workload": "%s shape (%d x %d x %d), width %d, %s" % (w.name, w.batch, w.dim, w.seqlen, K, w.io),
           "rotated_input_sets": R, "launch_ms": mean, "launch_ms_median": ms[n // 2],
           "roofline": {"bound": "hbm", "achieved": b / (mean * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": b / (mean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "traffic": traffic_from_profile("conv_" + w.name, 1), "algorithmic_bytes_per_launch": b}}

    wd = W.WORKLOADS["decode2p8b"]
    steps = min(args.decode_steps, 200)
    wt, bias = W.conv_params(wd, K, device="cuda")
    per_state = 2 * wd.batch * wd.dim * (K - 1)
    nstate = max(1, math.ceil(1.25 * MALL_BYTES / per_state))
    states = [torch.zeros((wd.batch, wd.dim, K - 1), dtype=torch.bfloat16, device="cuda") for _ in range(nstate)]
    xs = [W.conv_decode_inputs(wd, k, device="cuda") for k in range(steps)]
    outs = [torch.empty(wd.batch, wd.dim, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for k in range(min(10, steps)):
        ssm.conv1d_update(states[k % nstate], xs[k], wt, bias, out=outs[k % 2])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(steps):
        ssm.conv1d_update(states[k % nstate], xs[k], wt, bias, out=outs[k % 2])
        ev[k + 1].record()
    torch.cuda.synchronize()
    eager_ms = ev[0].elapsed_time(ev[steps]) / steps
    # A step of this size runs for less time than a Python call takes to issue it, so the eager
    # loop measures the host.  The same launches captured once in a HIP graph and replayed
    # back to back measure the device.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for k in range(steps):
                ssm.conv1d_update(states[k % nstate], xs[k], wt, bias, out=outs[k % 2])
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    gpu_ms = g0.elapsed_time(g1) / steps
    bd = conv_step_bytes(wd, K)
    dec = {"workload": "%s shape (%d x %d), width %d, bf16" % (wd.name, wd.batch, wd.dim, K), "steps": steps,
           "rotated_state_buffers": nstate, "gpu_ms_per_step": gpu_ms, "timing": "HIP graph of the steps, replayed",
           "eager_ms_per_step": eager_ms,
           "roofline": {"bound": "hbm", "achieved": bd / (gpu_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": bd / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "traffic": traffic_from_profile("conv_update_" + wd.name, 1),
                        "algorithmic_bytes_per_step": bd}}
    return pre, dec


def copy_peak(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate (torch copy_ of nbytes): read + write bytes per second."""
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, x, w, seconds):
    """The fp64 oracle as it stands, on this host's cores, over the same inputs (repeated to ~seconds)."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import oracle

    host = {k: (None if v is None else np.ascontiguousarray(v.detach().to("cpu", torch.float64).numpy()))
            for k, v in x.items() if k not in ("out", "fs")}
    B_rows = w.batch
    upd = 0
    t0 = time.perf_counter()
    runs = 0
    while True:
        oracle.scan(host["u"], host["delta"], host["A"], host["B"], host["C"], D=host["D"], z=host["z"],
                    delta_bias=host["delta_bias"])
        upd += w.batch * w.dim * w.dstate * w.seqlen
        runs += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cores = oracle.max_threads()
    t1 = time.perf_counter()
    oracle.scan(host["u"], host["delta"], host["A"], host["B"], host["C"], D=host["D"], z=host["z"],
                delta_bias=host["delta_bias"], threads=1)
    one = w.batch * w.dim * w.dstate * w.seqlen / (time.perf_counter() - t1)
    return {"value": upd / dt, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "value_1_thread": one,
            "sample": "%d full pass(es) of the %s workload (%d x %d x %d x %d, the same bf16 inputs widened "
                      "to fp64), %.1f s wall" % (runs, w.name, B_rows, w.dim, w.dstate, w.seqlen, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba130m", choices=["mamba130m", "mamba1p3b", "dna1m", "tiny"])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan shards over (batch, channel) with no exchange, so "
              "no multi-GPU figure is produced (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy // 16
        src = torch.ones(n, 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 16, "launches": args.steps}))
        return
    sys.path.insert(0, ROOT)
    import selective_state_space_76_amd as ssm
    from selective_state_space_76_amd import workloads as W
    ssm.load()

    w, R, ms_step, launch_ms, all_launch, x0, flushed = bench_scan(args, torch, ssm, W)
    upd = w.updates
    b = scan_bytes(w)
    value = upd / (ms_step * 1e-3)
    alu = upd * OPS_PER_UPDATE / (launch_ms * 1e-3) / 1e12
    gbs = b / (launch_ms * 1e-3) / 1e9
    log("scan: %.4f ms/step (wall), %.4f ms/launch (events) -> %.3e updates/s, %.1f GB/s"
        % (ms_step, launch_ms, value, gbs))
    res = {
        "metric": METRIC, "value": value, "unit": "state-updates/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen,
                   "io_dtype": w.io, "state_dtype": "f32", "rotated_input_sets": R},
        "roofline": {"bound": "alu", "achieved": alu, "peak": ALU_PEAK_TOPS, "unit": "T fp32-op/s",
                     "frac": alu / ALU_PEAK_TOPS, "traffic": traffic_from_profile(w.name, 1),
                     "ops_per_update": OPS_PER_UPDATE, "launch_ms": launch_ms,
                     "launch_ms_median": all_launch[len(all_launch) // 2],
                     "launch_ms_p10": all_launch[len(all_launch) // 10],
                     "launch_ms_p90": all_launch[(9 * len(all_launch)) // 10],
                     "flushed_launch_ms_median": flushed[len(flushed) // 2],
                     "flushed_launch_ms_p10": flushed[len(flushed) // 10],
                     "flushed_launch_ms_p90": flushed[(9 * len(flushed)) // 10]},
        "hbm": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "algorithmic_bytes_per_launch": b},
        "kernel_source_hash": kernel_source_hash(),
        "input_fp64_sums": {k: float(v.double().sum()) for k, v in x0.items()
                            if v is not None and k not in ("out", "fs")},
        "input_hash64": {k: hashlib.blake2b(v.contiguous().view(torch.uint8).cpu().numpy().tobytes(),
                                            digest_size=8).hexdigest()
                         for k, v in x0.items() if v is not None and k not in ("out", "fs")},
    }
    cp = copy_peak(torch)
    res["hbm"]["copy_peak_GBs"] = cp
    res["hbm"]["frac_of_copy_peak"] = gbs / cp
    log("device copy (torch copy_, 1 GiB): %.1f GB/s" % cp)
    if not args.no_decode:
        d = bench_decode(args, torch, ssm, W)
        log("decode: %.4f ms/step eager wall, %.4f ms/step eager events, %.4f ms/step graph, %.1f GB/s"
            % (d["eager_wall_ms_per_step"], d["eager_gpu_ms_per_step"], d["gpu_ms_per_step"], d["roofline"]["achieved"]))
        res["decode"] = d
        d["roofline"]["frac_of_copy_peak"] = d["roofline"]["achieved"] / cp
    if not args.no_bwd:
        bw = bench_bwd(args, torch, ssm, W)
        log("backward: %.4f ms/call -> %.3e updates/s (from saved checkpoints %.4f ms, ZOH %.4f ms)"
            % (bw["call_ms"], bw["value"], bw["from_saved_checkpoints_call_ms"], bw["zoh_call_ms"]))
        res["backward"] = bw
    if not args.no_conv:
        pre, dec = bench_conv(args, torch, ssm, W)
        log("conv1d: %.4f ms/launch, %.1f GB/s; conv1d_update: %.4f ms/step, %.1f GB/s"
            % (pre["launch_ms"], pre["roofline"]["achieved"], dec["gpu_ms_per_step"], dec["roofline"]["achieved"]))
        pre["roofline"]["frac_of_copy_peak"] = pre["roofline"]["achieved"] / cp
        dec["roofline"]["frac_of_copy_peak"] = dec["roofline"]["achieved"] / cp
        res["conv1d"] = pre
        res["conv1d_update"] = dec
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(torch, x0, w, args.cpu_seconds)
        log("cpu baseline: %.3e updates/s on %d threads" % (res["cpu_baseline"]["value"], res["cpu_baseline"]["cores"]))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
