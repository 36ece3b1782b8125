#!/usr/bin/env python3
"""Throughput of the MI355X selective scan (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dna1m]

A step is one ssm_scan_fwd call over a whole batch of the workload (discretise,
scan, carry across sequence segments, output epilogue: the entire
prefill/training-forward path) with every input already resident in HBM.  The
headline workload is the largest configuration, the million-step DNA-like
sequence (1 x 1024 channels x 16 states x 1,048,576 steps); the 130M- and
1.3B-shaped layer scans are measured the same way as sub-records.  Inputs are
rotated through enough independent sets that they cannot be served from the
256 MB Infinity Cache.  The same JSON line carries the decode path
(ssm_state_update) on the 2.8B-shaped generation workload, the backward pass
(ssm_scan_bwd) on the two layer shapes, the conv + SiLU step that produces u,
the 130M-shaped scan in the time-parallel layout beside the library's (the
layout comparison), a probe of the VALU issue rate, and the fp64 CPU oracle's
rate on a bounded sample of the headline workload.

Progress goes to stderr; stdout gets exactly one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "selective-scan state updates/sec (B·L·D·N) and HBM GB/s % of peak, 1 MI355X"
HBM_PEAK_GBS = 8000.0
# Published MI355X fp32 vector peak (it counts packed two-per-lane FMAs; see alu_issue_probe).
FP32_PEAK_TFLOPS = 157.3
# Algorithmic fp32 work of one forward state update: the exp2 argument (mul), exp2, B_bar * u
# (mul), the state update (FMA) and C * h (FMA); multiplies and the exp count 1, FMAs 2.
FLOPS_PER_UPDATE = 7
# Backward, per state update: restore the state (exp argument, exp, B_bar * u, FMA: 5); the adjoint
# G = G * A_bar + dy * C (mul + FMA: 3); dC += dy * h and dB += G * dt * u, each a product added
# over channels (2 + 2); sum_n G * B (FMA: 2); p = h_prev * A_bar, q = G * p, ddt += q * A (FMA),
# dA += q * dt (FMA) (1 + 1 + 2 + 2).
BWD_FLOPS_PER_UPDATE = 20
MALL_BYTES = 256 << 20
SUB_CONFIGS = ("mamba130m", "mamba1p3b")


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


def scan_record(args, torch, ssm, W, name, steps, warmup, keep_inputs=False):
    """Time ssm_scan_fwd on one workload: events around every call on the launch stream (torch's
    current stream), wall time over all calls.  Returns the record (and the first input set)."""
    w = W.WORKLOADS[name]
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
    io = ssm.SSM_BF16 if w.io == "bf16" else ssm.SSM_F32
    need = ssm.workspace_size(w.batch, w.dim, w.dstate, w.seqlen, io)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None

    def call(x):
        ssm.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                     out=x["out"], final_state=x["fs"], workspace=ws)

    for k in range(warmup):
        call(sets[k % R])
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        starts[k].record()
        call(sets[k % R])
        ends[k].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launch = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))
    ms_step = (t1 - t0) * 1e3 / steps
    mean = sum(launch) / len(launch)
    rec = {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen,
           "io_dtype": w.io, "rotated_input_sets": R, "steps": steps, "ms_per_step": ms_step,
           "value": w.updates / (ms_step * 1e-3), "unit": "state-updates/s",
           "call_ms": mean, "call_ms_median": launch[len(launch) // 2],
           "call_ms_p10": launch[len(launch) // 10], "call_ms_p90": launch[(9 * len(launch)) // 10],
           "workspace_bytes": need}
    if R > 1 and per_set <= MALL_BYTES:
        # the same call with L2 and the Infinity Cache flushed before each rep (a 1 GiB fill outside
        # the events), as a cross-check of the rotation above
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        nf = min(steps, 20)
        fs_ = [torch.cuda.Event(enable_timing=True) for _ in range(nf)]
        fe_ = [torch.cuda.Event(enable_timing=True) for _ in range(nf)]
        for k in range(nf):
            flush.zero_()
            fs_[k].record()
            call(sets[k % R])
            fe_[k].record()
        torch.cuda.synchronize()
        flushed = sorted(a.elapsed_time(b) for a, b in zip(fs_, fe_))
        del flush
        rec["flushed_call_ms_median"] = flushed[len(flushed) // 2]
    flops = w.updates * FLOPS_PER_UPDATE / (mean * 1e-3) / 1e12
    b = scan_bytes(w)
    gbs = b / (mean * 1e-3) / 1e9
    rec["roofline"] = {"bound": "alu", "achieved": flops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": flops / FP32_PEAK_TFLOPS, "traffic": traffic_from_profile(w.name, 1),
                       "flops_per_update": FLOPS_PER_UPDATE, "algorithmic_flops_per_call": w.updates * FLOPS_PER_UPDATE,
                       "call_ms": mean}
    rec["hbm"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                  "algorithmic_bytes_per_call": b}
    log("scan %s: %.4f ms/step (wall), %.4f ms/call (events) -> %.3e updates/s, %.2f TFLOP/s, %.1f GB/s"
        % (w.name, ms_step, mean, rec["value"], flops, gbs))
    x0 = sets[0] if keep_inputs else None
    del sets, ws
    return rec, w, x0


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


def bench_bwd(args, torch, ssm, W, name):
    """One ssm_scan_bwd call per step on a layer workload (checkpoint pass, backward pass and
    the fixed-order partial sums), inputs rotated past the Infinity Cache."""
    w = W.WORKLOADS[name]
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
    flops = w.updates * BWD_FLOPS_PER_UPDATE / (mean * 1e-3) / 1e12
    gbs = b / (mean * 1e-3) / 1e9
    rec = {"workload": w.name, "rotated_input_sets": R, "call_ms": mean, "call_ms_median": ms[n // 2],
           "value": w.updates / (mean * 1e-3), "unit": "state-updates/s", "workspace_bytes": need,
           "roofline": {"bound": "alu", "achieved": flops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": flops / FP32_PEAK_TFLOPS, "flops_per_update": BWD_FLOPS_PER_UPDATE,
                        "traffic": traffic_from_profile("bwd_" + w.name, 1), "call_ms": mean},
           "hbm": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                   "algorithmic_bytes_per_call": b},
           "zoh_call_ms": sum(mz) / len(mz), "from_saved_checkpoints_call_ms": sum(msv) / len(msv)}
    log("backward %s: %.4f ms/call -> %.3e updates/s, %.2f TFLOP/s (from saved checkpoints %.4f ms, ZOH %.4f ms)"
        % (w.name, mean, rec["value"], flops, rec["from_saved_checkpoints_call_ms"], rec["zoh_call_ms"]))
    del sets, ws, grads
    return rec


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


def bench_conv(args, torch, ssm, W, K=4, name="mamba130m"):
    """The conv + SiLU step that produces u, on a layer workload's [B, D, L] shape, and its
    decode form on the generation workload; events bracket each launch on the launch stream."""
    w = W.WORKLOADS[name]
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


def cpu_baseline(torch, x, w, seconds, rows=128):
    """The fp64 oracle as it stands, on this host's cores (its OpenMP default), over a bounded
    sample of the same inputs: the first `rows` channels of batch row 0 over the whole sequence
    (repeated to ~seconds); also one thread on 4 channels."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import oracle

    rows = min(rows, w.dim)

    def take(t, nrow):
        if t is None:
            return None
        if t.dim() == 3 and t.shape[1] == w.dim and t.shape[2] == w.seqlen:  # [B, D, L] streams
            t = t[:1, :nrow]
        elif t.dim() == 3:  # B, C [B, N, L]
            t = t[:1]
        elif t.dim() == 2:  # A [D, N]
            t = t[:nrow]
        else:  # D, bias [D]
            t = t[:nrow]
        return np.ascontiguousarray(t.detach().to("cpu", torch.float64).numpy())

    def run(nrow, threads, budget):
        h = {k: take(v, nrow) for k, v in x.items() if k not in ("out", "fs")}
        upd, runs = 0, 0
        t0 = time.perf_counter()
        while True:
            oracle.scan(h["u"], h["delta"], h["A"], h["B"], h["C"], D=h["D"], z=h["z"],
                        delta_bias=h["delta_bias"], threads=threads)
            upd += nrow * w.dstate * w.seqlen
            runs += 1
            if time.perf_counter() - t0 >= budget:
                break
        return upd / (time.perf_counter() - t0), runs, time.perf_counter() - t0

    v, runs, dt = run(rows, 0, seconds)
    one, _, _ = run(4, 1, 0.0)
    return {"value": v, "unit": "state-updates/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "value_1_thread": one,
            "sample": "%d pass(es) over the first %d channels of the %s workload (1 x %d x %d x %d: all %d steps, "
                      "the same bf16 inputs widened to fp64), %.1f s wall; one thread: 4 channels"
                      % (runs, rows, w.name, rows, w.dstate, w.seqlen, w.seqlen, dt)}


def issue_probe():
    """Measured issue rates, 8 waves per SIMD, from the probe library built beside the scan library
    (None if it is not built): plain wave64 fp32 work (v_fma_f32), v_exp_f32, and a multiply with a
    DPP row-broadcast operand."""
    path = os.path.join(ROOT, "selective_state_space_76_amd", "libssmprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.ssm_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.ssm_probe_issue.restype = ctypes.c_int
    res = {}
    for kind, name in ((0, "v_fma_f32"), (1, "v_exp_f32"), (2, "v_mul_f32_dpp_row_bcast")):
        clk, ms = ctypes.c_double(), ctypes.c_double()
        if lib.ssm_probe_issue(kind, 8, 1000, 2.4, ctypes.byref(clk), ctypes.byref(ms)) != 0:
            return None
        res[name] = clk.value
    lanes = 1024 * 64 * 2.4e9  # SIMDs x lanes x clock
    return {"clk_per_wave64_instr_at_2p4GHz": res, "waves_per_simd": 8,
            "fma_tflops": 2 * lanes / res["v_fma_f32"] / 1e12, "exp_per_s": lanes / res["v_exp_f32"],
            "note": "fp32 FMA issue rate of the whole GPU, unpacked (against the published 157.3 TFLOP/s); "
                    "v_exp_f32 and DPP-sourced operations issue at a fraction of it"}


def tp_library():
    """The scan in the time-parallel layout, built beside the scan library (None if it is not built)."""
    path = os.path.join(ROOT, "selective_state_space_76_amd", "libssmtp.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.ssm_tp_scan_fwd.argtypes = [i64, i64, i64, i64] + [vp] * 12
    lib.ssm_tp_scan_fwd.restype = ctypes.c_int
    return lib


def tp_scan_fwd(torch, lib, g, out, final_state=None, init=None):
    """out (and final_state) from the time-parallel scan on torch's current stream; g holds the
    scan inputs as device tensors (bf16 streams)."""
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    Bsz, Dm, L = g["u"].shape
    rc = lib.ssm_tp_scan_fwd(Bsz, Dm, g["A"].shape[1], L, p(g["u"]), p(g["delta"]), p(g["A"]), p(g["B"]),
                             p(g["C"]), p(g.get("D")), p(g.get("z")), p(g.get("delta_bias")), p(init), p(out),
                             p(final_state), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError("ssm_tp_scan_fwd returned %d" % rc)


def bench_layouts(torch, ssm, W, name="mamba130m", calls=20):
    """The library's scan against the same scan in the time-parallel layout (the pages' associative
    scan over time), same inputs, HIP events around each call."""
    lib = tp_library()
    if lib is None:
        return None
    w = W.WORKLOADS[name]
    g = W.scan_inputs(w, device="cuda")
    out = torch.empty_like(g["u"])
    fs = torch.empty(w.batch, w.dim, w.dstate, device="cuda")
    runs = {
        "library": lambda: ssm.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"],
                                        out=out, final_state=fs),
        "time_parallel": lambda: tp_scan_fwd(torch, lib, g, out, fs),
    }
    res = {"workload": "%s shape (%d x %d x %d x %d), bf16" % (name, w.batch, w.dim, w.dstate, w.seqlen)}
    for k, f in runs.items():
        for _ in range(3):
            f()
        ts = []
        for _ in range(calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        res[k + "_call_ms_median"] = ts[len(ts) // 2]
    res["note"] = ("the time-parallel layout: lanes over time, a row_shr DPP scan of (A_bar, B_bar u) pairs "
                   "over each row, states in a loop; the library keeps states on lanes and time sequential")
    return res


def input_digest(torch, x):
    """fp64 sums of every input and a 64-bit hash of its first 16 MiB (its bytes as stored)."""
    sums, hashes = {}, {}
    for k, v in x.items():
        if v is None or k in ("out", "fs"):
            continue
        sums[k] = float(v.double().sum())
        raw = v.contiguous().view(-1).view(torch.uint8)[: 16 << 20]
        hashes[k] = hashlib.blake2b(raw.cpu().numpy().tobytes(), digest_size=8).hexdigest()
    return sums, hashes


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dna1m", choices=["dna1m", "mamba130m", "mamba1p3b", "tiny"],
                    help="headline scan workload (default: the largest, dna1m)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-configs", action="store_true", help="skip the layer-shape scan sub-records")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-layout", action="store_true", help="skip the time-parallel layout comparison")
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

    head, w, x0 = scan_record(args, torch, ssm, W, args.workload, args.steps, args.warmup, keep_inputs=True)
    sums, hashes = input_digest(torch, x0)
    io = ssm.SSM_BF16 if w.io == "bf16" else ssm.SSM_F32
    res = {
        "metric": METRIC, "value": head["value"], "unit": "state-updates/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen,
                   "io_dtype": w.io, "state_dtype": "f32", "rotated_input_sets": head["rotated_input_sets"],
                   "workspace_bytes": ssm.workspace_size(w.batch, w.dim, w.dstate, w.seqlen, io)},
        "roofline": head["roofline"],
        "hbm": head["hbm"],
        "call_ms": head["call_ms"], "call_ms_median": head["call_ms_median"],
        "call_ms_p10": head["call_ms_p10"], "call_ms_p90": head["call_ms_p90"],
        "kernel_source_hash": kernel_source_hash(),
        "input_fp64_sums": sums, "input_hash64_first16MiB": hashes,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(torch, x0, w, args.cpu_seconds)
        log("cpu baseline: %.3e updates/s on %d threads (%s)" % (res["cpu_baseline"]["value"],
                                                                  res["cpu_baseline"]["cores"],
                                                                  res["cpu_baseline"]["sample"]))
    del x0
    torch.cuda.empty_cache()
    cp = copy_peak(torch)
    res["hbm"]["copy_peak_GBs"] = cp
    res["hbm"]["frac_of_copy_peak"] = res["hbm"]["achieved"] / cp
    log("device copy (torch copy_, 1 GiB): %.1f GB/s" % cp)
    if not args.no_configs:
        res["configs"] = {}
        for name in SUB_CONFIGS:
            if name == w.name:
                continue
            rec, _, _ = scan_record(args, torch, ssm, W, name, max(args.steps, 20), max(args.warmup, 3))
            rec["hbm"]["frac_of_copy_peak"] = rec["hbm"]["achieved"] / cp
            res["configs"][name] = rec
            torch.cuda.empty_cache()
    if not args.no_decode:
        d = bench_decode(args, torch, ssm, W)
        log("decode: %.4f ms/step eager wall, %.4f ms/step eager events, %.4f ms/step graph, %.1f GB/s"
            % (d["eager_wall_ms_per_step"], d["eager_gpu_ms_per_step"], d["gpu_ms_per_step"], d["roofline"]["achieved"]))
        res["decode"] = d
        d["roofline"]["frac_of_copy_peak"] = d["roofline"]["achieved"] / cp
        torch.cuda.empty_cache()
    if not args.no_bwd:
        res["backward"] = {}
        for name in SUB_CONFIGS:
            res["backward"][name] = bench_bwd(args, torch, ssm, W, name)
            torch.cuda.empty_cache()
    if not args.no_conv:
        pre, dec = bench_conv(args, torch, ssm, W)
        log("conv1d: %.4f ms/launch, %.1f GB/s; conv1d_update: %.4f ms/step, %.1f GB/s"
            % (pre["launch_ms"], pre["roofline"]["achieved"], dec["gpu_ms_per_step"], dec["roofline"]["achieved"]))
        pre["roofline"]["frac_of_copy_peak"] = pre["roofline"]["achieved"] / cp
        dec["roofline"]["frac_of_copy_peak"] = dec["roofline"]["achieved"] / cp
        res["conv1d"] = pre
        res["conv1d_update"] = dec
    if not args.no_layout:
        lay = bench_layouts(torch, ssm, W)
        if lay is not None:
            res["layout_alternative"] = lay
            log("layouts (%s): library %.4f ms, time-parallel %.4f ms per call"
                % (lay["workload"], lay["library_call_ms_median"], lay["time_parallel_call_ms_median"]))
        torch.cuda.empty_cache()
    if not args.no_probe:
        pr = issue_probe()
        if pr is not None:
            res["alu_issue_probe"] = pr
            log("issue probe: %s clk per wave64 instruction per SIMD" % pr["clk_per_wave64_instr_at_2p4GHz"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
