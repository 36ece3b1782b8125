"""Helpers for the GPU parity tests: the tolerance metric and oracle calls on sampled rows."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL_F32 = 1e-4   # fp32 streams
TOL_BF16 = 2e-2  # bf16 streams


def rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max(|ref_i|, rms(ref)): relative error with an RMS floor so that
    outputs near zero (gate ~ 0, cancellation over states) do not blow it up."""
    g = np.asarray(got.detach().to("cpu", torch.float64) if isinstance(got, torch.Tensor) else got, np.float64)
    r = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    den = np.maximum(np.abs(r), max(rms, 1e-300))
    return float(np.max(np.abs(g - r) / den)) if r.size else 0.0


def bf16_rne(x):
    """float64 values rounded to the nearest bfloat16 (ties to even), exactly; returned as float64."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def bf16_ulps(got, ref):
    """Distance in bf16 ulps between bf16 results and the exact values rounded to bf16."""
    g = got.detach().to("cpu").contiguous().view(torch.int16).numpy().astype(np.int32)
    r = torch.from_numpy(bf16_rne(ref).astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    r = r.numpy().astype(np.int32)

    def order(b):  # sign-magnitude bit patterns to a monotone integer scale
        return np.where(b < 0, -(b & 0x7FFF), b)
    return np.abs(order(g) - order(r))


ULP_SMALL_ABS = 2.0 ** -16  # absolute allowance for fp32 cancellation, as a fraction of rms(ref)


def check_bf16_ulp(got, ref, what=""):
    """bf16 results within one bf16 ulp of the fp64 result rounded to bf16 (RNE), or within
    ULP_SMALL_ABS * rms(ref) of the fp64 result.  A result is rounded once from fp32, so one ulp
    holds wherever the fp32 arithmetic before the rounding errs by less than an ulp of the element.
    An element much smaller than the terms it sums (the sum over states, an adjoint term) keeps
    the fp32 error of those terms, of order eps32 times their size, which exceeds an ulp of the
    element itself; the absolute allowance covers that.  For elements of at least 2^-8 rms(ref)
    one ulp is already above the allowance, so there the test is one ulp.  fp32 results are not
    checked here."""
    if got.dtype != torch.bfloat16:
        return
    r = np.asarray(ref, np.float64).reshape(tuple(got.shape))
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    d = bf16_ulps(got, r)
    g = got.detach().to("cpu", torch.float64).numpy()
    err = np.abs(g - r) / max(rms, 1e-300)
    allowed = err <= ULP_SMALL_ABS
    bad = (d > 1) & ~allowed
    big = np.abs(r) >= 2.0 ** -8 * rms
    worst = int(d[big].max()) if big.any() else 0
    print("%s bf16 ulps: max %d over %d elements >= 2^-8 rms (%d at 1 ulp); %d smaller elements more than "
          "1 ulp off, max err %.2g rms" % (what, worst, int(big.sum()), int((d[big] == 1).sum()),
                                           int(((d > 1) & ~big).sum()), float(err[(d > 1) & ~big].max())
                                           if ((d > 1) & ~big).any() else 0.0), flush=True)
    assert not bad.any(), (what, int(d[bad].max()), float(err[bad].max()))


def tol_for(x: torch.Tensor) -> float:
    return TOL_F32 if x.dtype == torch.float32 else TOL_BF16


def host(x):
    return None if x is None else x.detach().to("cpu")


def oracle_rows(inp, rows, h0=None, zoh=False, reverse=False):
    """Oracle on a subset of (b, d) rows: returns (out [R, L], final_state [R, N])."""
    outs, states = [], []
    by_b = {}
    for (b, d) in rows:
        by_b.setdefault(b, []).append(d)
    res = {}
    for b, ds in by_b.items():
        ds_t = torch.tensor(ds, device=inp["u"].device)
        sel = lambda t: None if t is None else host(t[b:b + 1].index_select(1, ds_t))
        o, s = oracle.scan(sel(inp["u"]), sel(inp["delta"]), host(inp["A"].index_select(0, ds_t)),
                           host(inp["B"][b:b + 1]), host(inp["C"][b:b + 1]),
                           D=None if inp.get("D") is None else host(inp["D"].index_select(0, ds_t)),
                           z=sel(inp.get("z")),
                           delta_bias=None if inp.get("delta_bias") is None else host(inp["delta_bias"].index_select(0, ds_t)),
                           h0=None if h0 is None else host(h0[b:b + 1].index_select(1, ds_t)),
                           zoh=zoh, reverse=reverse)
        for k, d in enumerate(ds):
            res[(b, d)] = (o[0, k], s[0, k])
    for key in rows:
        outs.append(res[key][0])
        states.append(res[key][1])
    return np.stack(outs), np.stack(states)


def sample_rows(Bsz, Dm, count, seed=0):
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (Bsz - 1, Dm - 1), (0, Dm - 1), (Bsz - 1, 0)}
    while len(rows) < min(count, Bsz * Dm):
        rows.add((int(rng.integers(Bsz)), int(rng.integers(Dm))))
    return sorted(rows)
