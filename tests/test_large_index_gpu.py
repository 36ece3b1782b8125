"""Tensors of more than 2^31 elements (GPU): 64-bit addressing in every kernel.

The [B, D, L] streams of the scan, its backward and the conv (8 x 8192 x 40000 bf16, 2.6e9
elements, 5.2 GB each), the decode state (4096 x 40960 x 16 fp32, 2.7e9 elements, 10.7 GB) and
the conv decode state (16384 x 49152 x 3 bf16, 2.4e9 elements) are indexed past 2^31 elements
and past 2^32 bytes.  The channels compared with the oracle are chosen at those boundaries:
for the scan row r = b D + d starts at element r L, so row 53687 (b 6, d 4535) straddles
element 2^31 and row 65535 (the last) starts at 2.6e9 elements, 5.2e9 bytes."""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_76_amd import conv1d_fwd, conv1d_update, scan_bwd, scan_fwd, state_update
from selective_state_space_76_amd import workloads as W
from tests.gpu_util import oracle_rows, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2  # bf16 streams


def _big_scan_workload():
    return W.WORKLOADS["mamba130m"].with_shape(batch=8, dim=8192, seqlen=40000, seed=9100)


def test_scan_and_backward_past_2_31_elements():
    w = _big_scan_workload()
    B, D, N, L = w.batch, w.dim, w.dstate, w.seqlen
    assert B * D * L > 2 ** 31 and (B * D - 1) * L * 2 > 2 ** 32
    print("case: scan %dx%dx%dx%d bf16 (%.2e elements per stream)" % (B, D, N, L, B * D * L), flush=True)
    x = W.scan_inputs(w, device=DEV)
    out, fs = scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
    torch.cuda.synchronize()
    rows = [(0, 0), (6, 4534), (6, 4535), (6, 4536), (7, 0), (7, 8191)]
    assert (6 * D + 4535) * L < 2 ** 31 < (6 * D + 4536) * L
    ref_y, ref_h = oracle_rows(x, rows)
    got_y = torch.stack([out[b, d] for b, d in rows])
    got_h = torch.stack([fs[b, d] for b, d in rows])
    ey, eh = rel_err(got_y, ref_y), rel_err(got_h, ref_h)
    print("forward rel_err y=%.3g state=%.3g" % (ey, eh), flush=True)
    assert ey <= TOL and eh <= TOL, (ey, eh)
    del out, fs

    print("case: backward of the same call", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(9101)
    dout = torch.randn(B, D, L, generator=g, device=DEV).to(torch.bfloat16)
    gr = scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], dout=dout)
    torch.cuda.synchronize()
    ci = torch.tensor([0, 4535, 4536, 8191], device=DEV)
    sel = lambda t: t.index_select(1, ci).cpu()
    selc = lambda t: t.index_select(0, ci).cpu()
    ref = oracle.scan_bwd(sel(x["u"]), sel(x["delta"]), selc(x["A"]), x["B"].cpu(), x["C"].cpu(), selc(x["D"]),
                          sel(x["z"]), selc(x["delta_bias"]), dout=sel(dout))
    got = {"du": sel(gr["du"]), "ddelta": sel(gr["ddelta"]), "dz": sel(gr["dz"]), "dA": selc(gr["dA"]),
           "dD": selc(gr["dD"]), "ddelta_bias": selc(gr["ddelta_bias"]), "dh0": sel(gr["dinitial_state"])}
    errs = {k: rel_err(v, ref[k]) for k, v in got.items() if v is not None and ref.get(k) is not None}
    print("backward sampled rel_err " + " ".join("%s=%.2g" % kv for kv in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL}
    assert not bad, bad
    assert torch.isfinite(gr["dB"]).all() and torch.isfinite(gr["dC"]).all()

    print("case: conv1d + SiLU on the same shape", flush=True)
    K = 4
    cw, cb = W.conv_params(w, K, device=DEV)
    u, cs = conv1d_fwd(x["u"], cw, cb)
    torch.cuda.synchronize()
    for b, d in rows:
        ru, rs = oracle.conv1d(x["u"][b:b + 1, d:d + 1].cpu(), cw[d:d + 1].cpu(), cb[d:d + 1].cpu())
        eu, es = rel_err(u[b:b + 1, d:d + 1], ru), rel_err(cs[b:b + 1, d:d + 1], rs)
        assert eu <= TOL and es <= TOL, ((b, d), eu, es)
    print("conv sampled rows within %g" % TOL, flush=True)


def test_decode_step_past_2_31_state_elements():
    w = W.WORKLOADS["decode2p8b"].with_shape(batch=4096, dim=40960, seed=9200)
    B, D, N = w.batch, w.dim, w.dstate
    assert B * D * N > 2 ** 31
    print("case: decode step %dx%dx%d (%.2e state elements)" % (B, D, N, B * D * N), flush=True)
    A, Dv, bias = W.params(w, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(9201)
    state = torch.randn(B, D, N, generator=g, device=DEV)
    # rows at the 2^30-element (2^32-byte) and 2^31-element boundaries and at the end
    rows = [(0, 0), (1638, 16383), (1638, 16384), (3276, 32767), (3276, 32768), (B - 1, D - 1)]
    assert (1638 * D + 16384) * N == 2 ** 30 and (3276 * D + 32768) * N == 2 ** 31
    bi = torch.tensor([b for b, _ in rows], device=DEV)
    di = torch.tensor([d for _, d in rows], device=DEV)
    before = state[bi, di].cpu()
    xs = W.decode_inputs(w, 0, device=DEV)
    y = state_update(state, xs["u"], xs["delta"], A, xs["B"], xs["C"], Dv, xs["z"], bias)
    torch.cuda.synchronize()
    for k, (b, d) in enumerate(rows):
        pick = lambda t: t[b:b + 1, d:d + 1].cpu()
        ry, rs = oracle.step(before[k].view(1, 1, N), pick(xs["u"]), pick(xs["delta"]), A[d:d + 1].cpu(),
                             xs["B"][b:b + 1].cpu(), xs["C"][b:b + 1].cpu(), D=Dv[d:d + 1].cpu(), z=pick(xs["z"]),
                             delta_bias=None if bias is None else bias[d:d + 1].cpu())
        ey, es = rel_err(y[b:b + 1, d:d + 1], ry), rel_err(state[b:b + 1, d:d + 1], rs)
        assert ey <= TOL and es <= TOL, ((b, d), ey, es)
    print("decode sampled rows within %g" % TOL, flush=True)


def test_conv_update_past_2_31_state_elements():
    w = W.WORKLOADS["decode2p8b"].with_shape(batch=16384, dim=49152, seed=9300)
    B, D, K = w.batch, w.dim, 4
    assert B * D * (K - 1) > 2 ** 31
    print("case: conv update %dx%d K=%d (%.2e state elements)" % (B, D, K, B * D * (K - 1)), flush=True)
    cw, cb = W.conv_params(w, K, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(9301)
    st = torch.randn(B, D, K - 1, generator=g, device=DEV).to(torch.bfloat16)
    xin = torch.randn(B, D, generator=g, device=DEV).to(torch.bfloat16)
    last = B * D - 1
    edge = (2 ** 31) // (K - 1)  # row whose state starts nearest below element 2^31
    rows = [(0, 0), divmod(edge, D), divmod(edge + 1, D), divmod(last, D)]
    assert edge * (K - 1) < 2 ** 31 <= (edge + 1) * (K - 1)
    bi = torch.tensor([b for b, _ in rows], device=DEV)
    di = torch.tensor([d for _, d in rows], device=DEV)
    before = st[bi, di].cpu()
    u = conv1d_update(st, xin, cw, cb)
    torch.cuda.synchronize()
    for k, (b, d) in enumerate(rows):
        ru, rs = oracle.conv_step(before[k].view(1, 1, K - 1), xin[b:b + 1, d:d + 1].cpu(), cw[d:d + 1].cpu(),
                                  cb[d:d + 1].cpu())
        eu = rel_err(u[b:b + 1, d:d + 1], ru)
        es = rel_err(st[b:b + 1, d:d + 1], rs)
        assert eu <= TOL and es <= TOL, ((b, d), eu, es)
    print("conv update sampled rows within %g" % TOL, flush=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_rows_of_2_24_steps_or_more(dtype):
    """Rows of 2^24 steps or more take the scan's element-load staging (the whole-piece staging's buffer
    resources span 8 rows of L elements, so the library keeps it below 2^24), through the sequence split,
    in both directions; every element is compared with the oracle."""
    L = (1 << 24) + 64
    name = "tiny" if dtype == torch.float32 else "mamba130m"
    w = W.WORKLOADS[name].with_shape(batch=1, dim=2, dstate=4, seqlen=L, seed=9200)
    x = W.scan_inputs(w)
    tol = 1e-4 if dtype == torch.float32 else TOL
    for rev in (False, True):
        print("case: rows of 2^24 + 64 steps, %s, reverse=%s" % (dtype, rev), flush=True)
        g = {k: (None if v is None else v.to(DEV)) for k, v in x.items()}
        out, fs = scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], reverse=rev)
        torch.cuda.synchronize()
        ref_y, ref_h = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                   delta_bias=x["delta_bias"], reverse=rev)
        ey, eh = rel_err(out, ref_y), rel_err(fs, ref_h)
        print("rel_err y=%.3g state=%.3g" % (ey, eh), flush=True)
        assert ey <= tol and eh <= tol
