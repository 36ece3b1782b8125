"""HIP scan and state update against the fp64 oracle (GPU).

Small shapes are compared element by element (several 64-step blocks, ragged
tails, every states-per-lane variant); the full-size workloads are run in the
launch configuration the benchmark times and compared on sampled channels,
which the oracle computes row by row."""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_76_amd import SSM_F32, scan_fwd, state_update, workspace_size
from selective_state_space_76_amd import workloads as W
from tests.gpu_util import check_bf16_ulp, oracle_rows, rel_err, sample_rows, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def full_check(inp, h0=None, zoh=False, reverse=False, split=True, tol=None):
    g = dev(inp)
    out, fs = scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g.get("D"), g.get("z"), g.get("delta_bias"),
                       None if h0 is None else h0.to(DEV), zoh=zoh, reverse=reverse, split=split)
    torch.cuda.synchronize()
    ref_y, ref_h = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp.get("D"), z=inp.get("z"),
                               delta_bias=inp.get("delta_bias"), h0=h0, zoh=zoh, reverse=reverse)
    tol = tol or tol_for(inp["u"])
    ey, eh = rel_err(out, ref_y), rel_err(fs, ref_h)
    print("rel_err y=%.3g state=%.3g tol=%g" % (ey, eh, tol), flush=True)
    assert ey <= tol and eh <= tol, (ey, eh)
    check_bf16_ulp(out, ref_y, "y")
    return out, fs


def make(Bsz, Dm, N, L, dtype=torch.bfloat16, seed=0, gate=True, skip=True, bias=True, recipe="base"):
    name = "tiny" if dtype == torch.float32 else "mamba130m"
    w = W.WORKLOADS[name].with_shape(batch=Bsz, dim=Dm, dstate=N, seqlen=L, seed=1000 + seed, bias=bias,
                                     recipe=recipe)
    x = W.scan_inputs(w)
    if not gate:
        x["z"] = None
    if not skip:
        x["D"] = None
    return x


def test_tiny_workload_fp32():
    print("case: tiny workload fp32 1x64x16x256", flush=True)
    full_check(W.scan_inputs(W.WORKLOADS["tiny"]))


@pytest.mark.parametrize("N", [16, 32, 64, 1, 5, 20, 40, 48])
def test_states_per_lane_variants(N):
    print("case: N=%d bf16 2x24x%dx300" % (N, N), flush=True)
    full_check(make(2, 24, N, 300, seed=N))


@pytest.mark.parametrize("L", [1, 7, 63, 64, 65, 129, 1000, 1001])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_ragged_lengths(L, dtype):
    print("case: L=%d %s" % (L, dtype), flush=True)
    full_check(make(3, 20, 16, L, dtype=dtype, seed=L))


@pytest.mark.parametrize("opts", [dict(gate=False), dict(skip=False), dict(bias=False),
                                  dict(gate=False, skip=False, bias=False)], ids=str)
def test_optional_operands(opts):
    print("case: optional operands %s" % opts, flush=True)
    full_check(make(2, 33, 16, 257, dtype=torch.float32, seed=7, **opts))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_initial_state(dtype):
    print("case: initial state %s" % dtype, flush=True)
    x = make(2, 40, 16, 200, dtype=dtype, seed=3)
    h0 = torch.randn(2, 40, 16, generator=torch.Generator().manual_seed(5))
    full_check(x, h0=h0)


@pytest.mark.parametrize("L", [4096, 5000, 6151])
def test_split_path(L):
    """Few channels, long sequence: summary + carry + output passes."""
    print("case: split L=%d" % L, flush=True)
    x = make(1, 40, 16, L, seed=L)
    assert workspace_size(1, 40, 16, L) > 0
    full_check(x)
    h0 = torch.randn(1, 40, 16, generator=torch.Generator().manual_seed(9))
    full_check(x, h0=h0)


def test_split_path_fp32_wide_state():
    print("case: split fp32 N=64", flush=True)
    full_check(make(1, 16, 64, 3000, dtype=torch.float32, seed=11))


@pytest.mark.parametrize("L", [40000, 100000, 200000, 450000, 1000000, 1500000])
def test_split_segment_counts(L):
    """Few channels, very long sequences: with one segment per 1024 steps here (40 to 1465 segments)
    the carry pass runs in each of its forms -- two levels with 4, 8, 16 or 32 segments per thread
    and 16 or 32 groups, and one chain per (channel, state) beyond 1024 segments -- from an initial
    state."""
    print("case: split segment count, fp32 1x3x5x%d" % L, flush=True)
    x = make(1, 3, 5, L, dtype=torch.float32, seed=L % 997)
    assert workspace_size(1, 3, 5, L, SSM_F32) > 4 * 15 * (L // 1024)  # the carries of every segment
    h0 = torch.randn(1, 3, 5, generator=torch.Generator().manual_seed(13))
    full_check(x, h0=h0)


@pytest.mark.parametrize("name", ["mamba130m", "mamba1p3b", "dna1m"])
def test_full_workload_sampled(name):
    """The full-size workload in the benchmark's launch configuration, checked on sampled channels."""
    w = W.WORKLOADS[name]
    print("case: full workload %s %s" % (name, (w.batch, w.dim, w.dstate, w.seqlen)), flush=True)
    g = W.scan_inputs(w, device=DEV)
    out, fs = scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(fs).all()
    rows = sample_rows(w.batch, w.dim, 8 if name == "dna1m" else 48, seed=1)
    ref_y, ref_h = oracle_rows(g, rows)
    got_y = torch.stack([out[b, d] for b, d in rows])
    got_h = torch.stack([fs[b, d] for b, d in rows])
    ey, eh = rel_err(got_y, ref_y), rel_err(got_h, ref_h)
    print("%s rel_err y=%.3g state=%.3g" % (name, ey, eh), flush=True)
    assert ey <= 2e-2 and eh <= 2e-2
    check_bf16_ulp(got_y, ref_y, name + " y")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 64, 6])
def test_state_update_small(dtype, N):
    print("case: state update N=%d %s" % (N, dtype), flush=True)
    w = W.WORKLOADS["decode2p8b"].with_shape(batch=3, dim=50, dstate=N)
    A, Dv, bias = W.params(w)
    state = torch.randn(3, 50, N, generator=torch.Generator().manual_seed(N))
    st = state.to(DEV)
    for k in range(5):
        x = W.decode_inputs(w, k)
        x = {kk: v.to(dtype) for kk, v in x.items()}
        y = state_update(st, x["u"].to(DEV), x["delta"].to(DEV), A.to(DEV), x["B"].to(DEV), x["C"].to(DEV),
                         Dv.to(DEV), x["z"].to(DEV), bias.to(DEV))
        torch.cuda.synchronize()
        ref_y, state = oracle.step(state, x["u"], x["delta"], A, x["B"], x["C"], D=Dv, z=x["z"], delta_bias=bias)
        tol = 1e-4 if dtype == torch.float32 else 2e-2
        ey, es = rel_err(y, ref_y), rel_err(st, state)
        assert ey <= tol and es <= tol, (k, ey, es)
        check_bf16_ulp(y, ref_y, "step %d y" % k)


def test_decode_workload_sampled():
    """decode2p8b: 1000 consecutive tokens from a zero state; a sampled grid of batch rows x channels
    follows the oracle's recurrence step by step."""
    w = W.WORKLOADS["decode2p8b"]
    print("case: decode workload %d steps" % w.steps, flush=True)
    A, Dv, bias = W.params(w, device=DEV)
    st = torch.zeros(w.batch, w.dim, w.dstate, device=DEV)
    bsel = torch.tensor([0, 77, 150, w.batch - 1], device=DEV)
    dsel = torch.tensor(sorted({0, 1, 15, 16, 17, 1023, 2500, 4096, w.dim - 1} |
                               set(np.random.default_rng(3).integers(0, w.dim, 7).tolist())), device=DEV)
    sub = lambda t: t.index_select(0, bsel).index_select(1, dsel).cpu()
    ref_state = np.zeros((len(bsel), len(dsel), w.dstate))
    A_h, D_h, bias_h = A[dsel].cpu(), Dv[dsel].cpu(), bias[dsel].cpu()
    worst = 0.0
    for k in range(w.steps):
        x = W.decode_inputs(w, k, device=DEV)
        y = state_update(st, x["u"], x["delta"], A, x["B"], x["C"], Dv, x["z"], bias)
        ref_y, ref_state = oracle.step(ref_state, sub(x["u"]), sub(x["delta"]), A_h, x["B"][bsel].cpu(),
                                       x["C"][bsel].cpu(), D=D_h, z=sub(x["z"]), delta_bias=bias_h)
        if k % 100 == 99 or k == 0:
            worst = max(worst, rel_err(sub(y), ref_y), rel_err(sub(st), ref_state))
            print("step %d worst rel_err %.3g" % (k, worst), flush=True)
            check_bf16_ulp(sub(y), ref_y, "step %d y" % k)
    assert worst <= 2e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("L", [300, 1000, 1001, 4500])
def test_zoh(dtype, L):
    """Exact zero-order-hold B_bar (the oracle's ZOH is pinned to scipy's cont2discrete)."""
    print("case: zoh L=%d %s" % (L, dtype), flush=True)
    x = make(1 if L > 4000 else 2, 40 if L > 4000 else 24, 16, L, dtype=dtype, seed=L + 1)
    full_check(x, zoh=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("L", [300, 1000, 1001, 4500])
def test_reverse(dtype, L):
    """Backward-in-time scan, with and without a sequence split and an initial state."""
    print("case: reverse L=%d %s" % (L, dtype), flush=True)
    x = make(1 if L > 4000 else 2, 40 if L > 4000 else 24, 16, L, dtype=dtype, seed=L + 2)
    full_check(x, reverse=True)
    h0 = torch.randn(x["u"].shape[0], x["u"].shape[1], 16, generator=torch.Generator().manual_seed(L))
    full_check(x, h0=h0, reverse=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("N", [32, 40, 64])
def test_zoh_state_slices(dtype, N):
    """ZOH with two and four state slices per lane, ragged length, with an initial state."""
    print("case: zoh N=%d %s 2x24x%dx1001" % (N, dtype, N), flush=True)
    x = make(2, 24, N, 1001, dtype=dtype, seed=300 + N)
    h0 = torch.randn(2, 24, N, generator=torch.Generator().manual_seed(N))
    full_check(x, h0=h0, zoh=True)


def test_zoh_split_wide_state():
    """ZOH through the sequence split (summary, carry and output passes) with 64 states."""
    print("case: zoh split N=64 1x40x64x4500", flush=True)
    full_check(make(1, 40, 64, 4500, seed=77), zoh=True)


def test_reverse_zoh_wide_state():
    print("case: reverse+zoh N=64", flush=True)
    full_check(make(2, 20, 64, 700, dtype=torch.float32, seed=99), zoh=True, reverse=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_state_update_zoh(dtype):
    print("case: state update zoh %s" % dtype, flush=True)
    w = W.WORKLOADS["decode2p8b"].with_shape(batch=3, dim=40, dstate=16)
    A, Dv, bias = W.params(w)
    state = torch.randn(3, 40, 16, generator=torch.Generator().manual_seed(4))
    st = state.to(DEV)
    for k in range(4):
        x = {kk: v.to(dtype) for kk, v in W.decode_inputs(w, k).items()}
        y = state_update(st, x["u"].to(DEV), x["delta"].to(DEV), A.to(DEV), x["B"].to(DEV), x["C"].to(DEV),
                         Dv.to(DEV), x["z"].to(DEV), bias.to(DEV), zoh=True)
        torch.cuda.synchronize()
        ref_y, state = oracle.step(state, x["u"], x["delta"], A, x["B"], x["C"], D=Dv, z=x["z"], delta_bias=bias,
                                   zoh=True)
        tol = 1e-4 if dtype == torch.float32 else 2e-2
        assert rel_err(y, ref_y) <= tol and rel_err(st, state) <= tol


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("N", [16, 64])
def test_zero_and_tiny_decay(zoh, N):
    """Some A entries exactly 0 (no decay: the state sums its inputs; under ZOH the factor's
    1/A is infinite and the series takes over) and others tiny, in the scan (whole and split
    sequence) and in the decode step."""
    print("case: A = 0 and A = -1e-4 entries, zoh=%d N=%d" % (zoh, N), flush=True)
    for L in (300, 4200):
        x = make(1, 24, N, L, dtype=torch.float32, seed=900 + N + L)
        A = x["A"].clone()
        A[::3, ::2] = 0.0
        A[1::3, 1::4] = -1e-4
        x["A"] = A
        full_check(x, zoh=zoh)
    w = W.WORKLOADS["decode2p8b"].with_shape(batch=3, dim=24, dstate=N, seed=950 + N)
    A = torch.full((24, N), -0.5)
    A[::3, ::2] = 0.0
    A[1::3, 1::4] = -1e-4
    s = W.decode_inputs(w, 0)
    st0 = torch.randn(3, 24, N, generator=torch.Generator().manual_seed(951))
    st = st0.to(DEV)
    y = state_update(st, s["u"].float().to(DEV), s["delta"].float().to(DEV), A.to(DEV), s["B"].float().to(DEV),
                     s["C"].float().to(DEV), zoh=zoh)
    torch.cuda.synchronize()
    ry, rst = oracle.step(st0.double(), s["u"].float(), s["delta"].float(), A, s["B"].float(), s["C"].float(), zoh=zoh)
    assert rel_err(y, ry) <= 1e-4 and rel_err(st, rst) <= 1e-4


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
def test_wide_step_sizes(zoh):
    """delta + bias spread over [-30, 30]: softplus from its exponential tail to the linear
    branch above 20 (dt = x there), decays from ~1 to exactly 0 in fp32, in the scan and the
    backward."""
    print("case: wide step sizes, zoh=%d" % zoh, flush=True)
    x = make(2, 20, 16, 400, dtype=torch.float32, seed=990 + zoh)
    g = torch.Generator().manual_seed(991)
    x["delta"] = (torch.rand(x["delta"].shape, generator=g) * 60.0 - 30.0).float()
    x["delta_bias"] = torch.zeros_like(x["delta_bias"])
    full_check(x, zoh=zoh)
    from selective_state_space_76_amd import scan_bwd
    d = dev(x)
    gr = scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"], dout=d["u"], zoh=zoh)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], None,
                          dout=x["u"], dfinal=None, zoh=zoh)
    errs = {k: rel_err(gr[k], ref[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias")}
    print("rel_err " + " ".join("%s=%.2g" % kv for kv in errs.items()), flush=True)
    assert all(e <= 1e-4 for e in errs.values()), errs


def _extreme(case):
    if case == "A_spread":          # decay factors from 0 (A = -1e4) to ~1 (A = -1e-6)
        x = make(2, 20, 16, 300, dtype=torch.float32, seed=1)
        A = x["A"].clone()
        A[:, ::3] = -1e4
        A[:, 1::3] = -1e-6
        x["A"] = A
    elif case == "large_u_BC":      # u x100, B and C x10
        x = make(2, 20, 16, 300, dtype=torch.float32, seed=2)
        x["u"], x["B"], x["C"] = x["u"] * 100.0, x["B"] * 10.0, x["C"] * 10.0
    elif case == "wide_gate":       # z over [-50, 50]: the gate from ~0 to the identity
        x = make(2, 20, 16, 300, dtype=torch.float32, seed=3)
        x["z"] = (torch.rand(x["z"].shape, generator=torch.Generator().manual_seed(4)) * 100.0 - 50.0).float()
    else:                           # tiny steps: dt ~ 6e-6
        x = make(1, 20, 16, 300, dtype=torch.float32, seed=5)
        x["delta_bias"] = torch.full_like(x["delta_bias"], -12.0)
    return x


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
@pytest.mark.parametrize("case", ["A_spread", "large_u_BC", "wide_gate", "tiny_steps"])
def test_extreme_magnitudes(case, zoh):
    """Finite but extreme inputs, scan and backward against the oracle at the fp32 tolerance."""
    print("case: extreme %s zoh=%d" % (case, zoh), flush=True)
    x = _extreme(case)
    full_check(x, zoh=zoh)
    from selective_state_space_76_amd import scan_bwd
    d = dev(x)
    gr = scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"], dout=d["u"], zoh=zoh)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], None,
                          dout=x["u"], dfinal=None, zoh=zoh)
    errs = {k: rel_err(gr[k], ref[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias")}
    print("rel_err " + " ".join("%s=%.2g" % kv for kv in errs.items()), flush=True)
    assert all(torch.isfinite(v).all() for v in gr.values() if v is not None)
    assert all(e <= 1e-4 for e in errs.values()), errs
