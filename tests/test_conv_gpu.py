"""HIP conv1d + SiLU (the step that produces u) against the fp64 oracle (GPU).

Small shapes cover every width, both dtypes, lengths that take the 16-byte-chunk
path and the per-element path (ragged tails, L below the width), with and
without a carried state; the workload shapes are compared in full or on sampled
channels.  Carried states are copies of inputs, so they must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_76_amd import conv1d_fwd, conv1d_update, scan_fwd
from selective_state_space_76_amd import workloads as W
from tests.gpu_util import check_bf16_ulp, rel_err, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make(Bsz, Dm, L, K, dtype, seed, state):
    name = "tiny" if dtype == torch.float32 else "mamba130m"
    w = W.WORKLOADS[name].with_shape(batch=Bsz, dim=Dm, seqlen=L, seed=2000 + seed)
    return W.conv_inputs(w, K, state=state)


def check(inp, bias=True, tol=None):
    x, wt = inp["x"], inp["weight"]
    b = inp["bias"] if bias else None
    st = inp.get("state")
    u, so = conv1d_fwd(x.to(DEV), wt.to(DEV), None if b is None else b.to(DEV),
                       None if st is None else st.to(DEV))
    torch.cuda.synchronize()
    ref_u, ref_s = oracle.conv1d(x, wt, b, st)
    e = rel_err(u, ref_u)
    tol = tol or tol_for(x)
    print("rel_err u=%.3g tol=%g" % (e, tol), flush=True)
    assert e <= tol, e
    check_bf16_ulp(u, ref_u, "u")
    assert np.array_equal(so.to("cpu", torch.float64).numpy(), ref_s)
    return u, so


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("L", [1, 2, 3, 5, 8, 9, 16, 63, 64, 100, 1000, 1024])
def test_conv_small(dtype, K, L):
    for state in (False, True):
        print("case: conv %s K=%d L=%d state=%s" % (dtype, K, L, state), flush=True)
        check(make(2, 37, L, K, dtype, seed=K * 100 + L, state=state), bias=not state or L % 2 == 0)


def test_conv_workload_mamba130m():
    w = W.WORKLOADS["mamba130m"]
    print("case: conv full 8x1536x2048 bf16 K=4", flush=True)
    check(W.conv_inputs(w, 4))


def test_conv_workload_dna1m_sampled():
    w = W.WORKLOADS["dna1m"]
    print("case: conv 1x1024x1048576 bf16 K=4, 8 channels compared", flush=True)
    inp = W.conv_inputs(w, 4, device=DEV)
    u, so = conv1d_fwd(inp["x"], inp["weight"], inp["bias"])
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 17, 255, 256, 600, 1022, 1023], device=DEV)
    ref_u, ref_s = oracle.conv1d(inp["x"].index_select(1, rows).cpu(), inp["weight"].index_select(0, rows).cpu(),
                                 inp["bias"].index_select(0, rows).cpu())
    e = rel_err(u.index_select(1, rows), ref_u)
    print("rel_err u=%.3g" % e, flush=True)
    assert e <= tol_for(u)
    check_bf16_ulp(u.index_select(1, rows), ref_u, "dna1m u")
    assert np.array_equal(so.index_select(1, rows).to("cpu", torch.float64).numpy(), ref_s)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_conv_pieces_equal_one_pass(dtype):
    """A sequence processed in pieces (state carried between two buffers) equals one pass,
    bit for bit, whichever kernel path each piece takes."""
    inp = make(3, 40, 1000, 4, dtype, seed=7, state=True)
    g = {k: v.to(DEV) for k, v in inp.items()}
    whole, s_whole = conv1d_fwd(g["x"], g["weight"], g["bias"], g["state"])
    cuts = [0, 1, 3, 8, 64, 65, 500, 1000]
    st = g["state"]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        u, st = conv1d_fwd(g["x"][..., a:b].contiguous(), g["weight"], g["bias"], st)
        parts.append(u)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=-1), whole)
    assert torch.equal(st, s_whole)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_update_chain(dtype, K):
    """50 decode steps from a random state: u against the oracle step by step, the state
    exactly, and the chain bitwise equal to one prefill over the same 50 inputs."""
    name = "tiny" if dtype == torch.float32 else "decode2p8b"
    w = W.WORKLOADS[name].with_shape(batch=8, dim=96, seqlen=1, seed=3000 + K)
    wt, b = W.conv_params(w, K)
    st0 = W.conv_inputs(w.with_shape(seqlen=1), K, state=True)["state"]
    xs = [W.conv_decode_inputs(w, t) for t in range(50)]
    st = st0.to(DEV).clone()
    ref_st = st0
    outs = []
    for t, xt in enumerate(xs):
        if t % 25 == 0:
            print("case: conv update %s K=%d step %d" % (dtype, K, t), flush=True)
        u = conv1d_update(st, xt.to(DEV), wt.to(DEV), b.to(DEV))
        torch.cuda.synchronize()
        ref_u, ref_st = oracle.conv_step(ref_st, xt, wt, b)
        assert rel_err(u, ref_u) <= tol_for(u)
        check_bf16_ulp(u, ref_u, "step %d u" % t)
        assert np.array_equal(st.to("cpu", torch.float64).numpy(), ref_st)
        outs.append(u)
    seq = torch.stack(xs, dim=-1).to(DEV)
    u_seq, s_seq = conv1d_fwd(seq, wt.to(DEV), b.to(DEV), st0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(outs, dim=-1), u_seq)
    assert torch.equal(s_seq, st)


def test_conv_update_workload_decode2p8b():
    w = W.WORKLOADS["decode2p8b"]
    print("case: conv update 256x5120 bf16 K=4, 3 steps", flush=True)
    wt, b = W.conv_params(w, 4, device=DEV)
    st = torch.zeros((w.batch, w.dim, 3), dtype=torch.bfloat16, device=DEV)
    ref_st = np.zeros((w.batch, w.dim, 3))
    for t in range(3):
        xt = W.conv_decode_inputs(w, t, device=DEV)
        u = conv1d_update(st, xt, wt, b)
        torch.cuda.synchronize()
        ref_u, ref_st = oracle.conv_step(ref_st, xt.cpu(), wt.cpu(), b.cpu())
        e = rel_err(u, ref_u)
        print("step %d rel_err u=%.3g" % (t, e), flush=True)
        assert e <= tol_for(u)
        check_bf16_ulp(u, ref_u, "step %d u" % t)
        assert np.array_equal(st.to("cpu", torch.float64).numpy(), ref_st)


def test_width1_ignores_state_pointers():
    inp = make(2, 16, 64, 1, torch.bfloat16, seed=11, state=False)
    g = {k: v.to(DEV) for k, v in inp.items()}
    u, so = conv1d_fwd(g["x"], g["weight"], g["bias"])
    ref_u, _ = oracle.conv1d(inp["x"], inp["weight"], inp["bias"])
    assert so.numel() == 0 and rel_err(u, ref_u) <= tol_for(u)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_conv_then_scan(dtype):
    """The two steps chained as in the pages' block: conv+SiLU produces u, the scan consumes it.
    The reference is the oracle's conv feeding the oracle's scan (in fp64 throughout, so the
    rounding of u to the stream dtype on the GPU side counts as error, well inside the bound)."""
    name = "tiny" if dtype == torch.float32 else "mamba130m"
    w = W.WORKLOADS[name].with_shape(batch=2, dim=48, dstate=16, seqlen=640, seed=4000)
    sc = W.scan_inputs(w)
    cv = W.conv_inputs(w, 4)
    g = {k: (None if v is None else v.to(DEV)) for k, v in sc.items()}
    u, _ = conv1d_fwd(cv["x"].to(DEV), cv["weight"].to(DEV), cv["bias"].to(DEV))
    out, fs = scan_fwd(u, g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"])
    torch.cuda.synchronize()
    ref_u, _ = oracle.conv1d(cv["x"], cv["weight"], cv["bias"])
    assert rel_err(u, ref_u) <= tol_for(u)
    ref_y, ref_h = oracle.scan(ref_u, sc["delta"], sc["A"], sc["B"], sc["C"], D=sc["D"], z=sc["z"],
                               delta_bias=sc["delta_bias"])
    ey, eh = rel_err(out, ref_y), rel_err(fs, ref_h)
    print("rel_err u-chain y=%.3g state=%.3g" % (ey, eh), flush=True)
    assert ey <= tol_for(u) and eh <= tol_for(u)
