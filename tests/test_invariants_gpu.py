"""Invariants of the HIP path that hold bit for bit or at any size (GPU)."""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_76_amd import scan_fwd, state_update, workspace_size
from selective_state_space_76_amd import workloads as W
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def inputs(Bsz, Dm, N, L, dtype=torch.bfloat16, seed=0, device=DEV):
    w = W.WORKLOADS["mamba130m"].with_shape(batch=Bsz, dim=Dm, dstate=N, seqlen=L, seed=5000 + seed)
    x = W.scan_inputs(w, device=device)
    if dtype == torch.float32:
        for k in ("u", "delta", "z", "B", "C"):
            x[k] = x[k].float()
    return x


def run(x, **kw):
    out, fs = scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], **kw)
    torch.cuda.synchronize()
    return out, fs


@pytest.mark.parametrize("shape", [(2, 40, 16, 1000), (1, 24, 16, 5000), (2, 20, 64, 700), (1, 64, 16, 4096)],
                         ids=str)
def test_deterministic(shape):
    print("case: determinism", shape, flush=True)
    x = inputs(*shape)
    o1, f1 = run(x)
    o2, f2 = run(x)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("shape", [(2, 40, 16, 1000), (1, 24, 16, 5000), (1, 64, 16, 4096)], ids=str)
@pytest.mark.parametrize("reverse", [False, True])
def test_causal_bitwise(shape, reverse):
    """Perturbing every input at step s leaves all outputs before s (after s when reversed) unchanged."""
    print("case: causality", shape, reverse, flush=True)
    x = inputs(*shape)
    o, _ = run(x, reverse=reverse)
    L = shape[3]
    for s in (1, 37, L // 2, L - 1):
        p = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        for k in ("u", "delta", "z", "B", "C"):
            p[k][..., s] += 0.75
        op, _ = run(p, reverse=reverse)
        if reverse:
            assert torch.equal(op[..., s + 1:], o[..., s + 1:])
            assert not torch.equal(op[..., s], o[..., s])
        else:
            assert torch.equal(op[..., :s], o[..., :s])
            assert not torch.equal(op[..., s], o[..., s])


def test_permutation_equivariance_bitwise():
    print("case: permutation", flush=True)
    x = inputs(3, 48, 16, 300)
    o, f = run(x)
    pd = torch.randperm(48, generator=torch.Generator().manual_seed(1)).to(DEV)
    pb = torch.tensor([2, 0, 1], device=DEV)
    p = dict(x)
    for k in ("u", "delta", "z"):
        p[k] = x[k][pb][:, pd].contiguous()
    for k in ("B", "C"):
        p[k] = x[k][pb].contiguous()
    p["A"] = x["A"][pd].contiguous()
    p["D"] = x["D"][pd].contiguous()
    p["delta_bias"] = x["delta_bias"][pd].contiguous()
    op, fp = run(p)
    assert torch.equal(op, o[pb][:, pd]) and torch.equal(fp, f[pb][:, pd])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("Dm", [32, 64], ids=["lanes_over_states", "channels_on_lanes"])
def test_split_matches_unsplit(dtype, Dm):
    """Few channels, long sequence: the three-pass split equals the single sequential pass (with bf16
    streams and D = 64 the split's passes keep channels on lanes)."""
    print("case: split vs unsplit", dtype, Dm, flush=True)
    x = inputs(1, Dm, 16, 9000, dtype=dtype, seed=3)
    assert workspace_size(1, Dm, 16, 9000) > 0
    o1, f1 = run(x)
    o2, f2 = run(x, split=False)
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    # outputs round to the stream dtype; compare both against each other in fp64
    assert rel_err(o1, o2.double().cpu().numpy()) <= tol
    assert rel_err(f1, f2.double().cpu().numpy()) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scan_equals_repeated_state_update(dtype):
    print("case: scan == L x state_update", dtype, flush=True)
    L = 48
    x = inputs(2, 40, 16, L, dtype=dtype, seed=4)
    o, f = run(x)
    st = torch.zeros(2, 40, 16, device=DEV)
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    for t in range(L):
        y = state_update(st, x["u"][..., t].contiguous(), x["delta"][..., t].contiguous(), x["A"],
                         x["B"][..., t].contiguous(), x["C"][..., t].contiguous(), x["D"],
                         x["z"][..., t].contiguous(), x["delta_bias"])
        assert rel_err(y, o[..., t].double().cpu().numpy()) <= tol, t
    torch.cuda.synchronize()
    assert rel_err(st, f.double().cpu().numpy()) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_chunked_calls_with_initial_state(dtype):
    """scan(x[:L1]) then scan(x[L1:], initial_state = its final state) == scan(x)."""
    print("case: chunking", dtype, flush=True)
    x = inputs(2, 36, 16, 2000, dtype=dtype, seed=5)
    o, f = run(x)
    L1 = 777
    part = lambda sl: {k: (v[..., sl].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
                       for k, v in x.items()}
    o1, f1 = run(part(slice(0, L1)))
    p2 = part(slice(L1, None))
    o2, f2 = scan_fwd(p2["u"], p2["delta"], p2["A"], p2["B"], p2["C"], p2["D"], p2["z"], p2["delta_bias"], f1)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    assert rel_err(torch.cat([o1, o2], -1), o.double().cpu().numpy()) <= tol
    assert rel_err(f2, f.double().cpu().numpy()) <= 1e-4
    # the same continuation in place: initial_state and final_state are one buffer
    h = f1.clone()
    scan_fwd(p2["u"], p2["delta"], p2["A"], p2["B"], p2["C"], p2["D"], p2["z"], p2["delta_bias"], h, final_state=h)
    torch.cuda.synchronize()
    assert torch.equal(h, f2)


def test_small_step_limit():
    """dt -> 0 (bias -40): out = D u silu(z) and the state stays ~0."""
    print("case: dt -> 0", flush=True)
    x = inputs(2, 40, 16, 300, dtype=torch.float32, seed=6)
    x["delta_bias"] = torch.full_like(x["delta_bias"], -40.0)
    o, f = run(x)
    ref = (x["D"][None, :, None] * x["u"] * torch.nn.functional.silu(x["z"])).double().cpu().numpy()
    assert rel_err(o, ref) <= 1e-5 and f.abs().max().item() < 1e-12


def test_full_workload_determinism_and_split_plan():
    """The DNA shape at 2^18 steps runs split (256 segments, channels on lanes); two runs agree bit
    for bit."""
    w = W.WORKLOADS["dna1m"].with_shape(seqlen=1 << 18)
    print("case: long split determinism", flush=True)
    x = W.scan_inputs(w, device=DEV)
    o1, f1 = run(x)
    o2, f2 = run(x)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_concurrent_streams_match_serial():
    """Calls on two streams at once (distinct outputs and workspaces, one split and one whole
    sequence, forward and backward) give the serial results bit for bit."""
    from selective_state_space_76_amd import scan_bwd
    xa = inputs(1, 24, 16, 5000, seed=31)   # split sequence
    xb = inputs(4, 256, 16, 1024, seed=32)  # whole sequence
    g = torch.Generator(device=DEV).manual_seed(33)
    for x in (xa, xb):
        x["dout"] = torch.randn(x["u"].shape, generator=g, device=DEV).to(x["u"].dtype)

    def work(x):
        out, fs = scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
        gr = scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], dout=x["dout"])
        return [out, fs] + [v for k, v in sorted(gr.items()) if v is not None]

    ref_a, ref_b = work(xa), work(xb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        print("case: two streams, repetition %d" % rep, flush=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            got_a = work(xa)
        with torch.cuda.stream(sb):
            got_b = work(xb)
        torch.cuda.synchronize()
        assert all(torch.equal(p, q) for p, q in zip(got_a, ref_a)), rep
        assert all(torch.equal(p, q) for p, q in zip(got_b, ref_b)), rep


def test_explicit_side_stream_with_internal_buffers():
    """stream= names a stream other than torch's current one, and the binding allocates the
    outputs and workspaces itself (on the current stream).  Right after each call the current
    stream allocates and overwrites memory of the same sizes; the side stream's results must
    still equal the serial ones bit for bit (the binding tells the allocator which stream uses
    the buffers it made)."""
    from selective_state_space_76_amd import scan_bwd
    x = inputs(1, 24, 16, 5000, seed=41)   # split sequence: forward and backward workspaces
    g = torch.Generator(device=DEV).manual_seed(42)
    x["dout"] = torch.randn(x["u"].shape, generator=g, device=DEV).to(x["u"].dtype)
    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
    ref_out, ref_fs = scan_fwd(*args)
    ref_g = scan_bwd(*args, dout=x["dout"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        print("case: side stream with internal buffers, repetition %d" % rep, flush=True)
        side.wait_stream(torch.cuda.current_stream())
        out, fs = scan_fwd(*args, stream=side)
        gr = scan_bwd(*args, dout=x["dout"], stream=side)
        # current-stream work that would land on any buffer handed back too early
        junk = [torch.full((n,), float("nan"), device=DEV) for n in (1 << 16, 1 << 20, 1 << 22, 1 << 24)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        assert torch.equal(out, ref_out) and torch.equal(fs, ref_fs), rep
        for k, v in ref_g.items():
            assert (v is None and gr[k] is None) or torch.equal(gr[k], v), (rep, k)
