"""Seeded input recipes: shapes, dtypes, value distributions and determinism (CPU)."""
import math

import numpy as np
import torch

from selective_state_space_76_amd import workloads as W


def small(name, **kw):
    return W.WORKLOADS[name].with_shape(**kw)


def test_shapes_and_dtypes():
    w = small("mamba130m", batch=2, dim=40, seqlen=300)
    x = W.scan_inputs(w)
    assert x["u"].shape == (2, 40, 300) and x["u"].dtype == torch.bfloat16
    assert x["B"].shape == (2, 16, 300) and x["C"].dtype == torch.bfloat16
    assert x["A"].shape == (40, 16) and x["A"].dtype == torch.float32
    assert x["D"].shape == (40,) and x["delta_bias"].shape == (40,)
    t = W.scan_inputs(W.WORKLOADS["tiny"])
    assert all(t[k].dtype == torch.float32 for k in ("u", "delta", "z", "B", "C"))
    assert W.WORKLOADS["mamba1p3b"].bias is False


def test_value_recipe():
    w = small("mamba130m", batch=2, dim=256, seqlen=1024)
    x = W.scan_inputs(w)
    u = x["u"].float()
    assert abs(u.mean().item()) < 0.02 and abs(u.std().item() - 1) < 0.02
    assert abs(x["delta"].float().std().item() - 0.5) < 0.01
    assert torch.equal(x["A"][:, 3], torch.full((256,), -4.0))
    assert torch.equal(x["D"], torch.ones(256))
    # dt_bias = softplus^-1(Delta*), Delta* in [1e-3, 1e-1]
    dstar = torch.nn.functional.softplus(x["delta_bias"].double())
    assert dstar.min() >= 1e-3 * (1 - 1e-5) and dstar.max() <= 1e-1 * (1 + 1e-5)
    # bf16 values are fp32 draws rounded once
    assert torch.equal(x["u"].float().to(torch.bfloat16), x["u"])


def test_logu_delta_recipe():
    w = small("mamba1p3b", batch=1, dim=64, seqlen=2048)
    x = W.scan_inputs(w)
    assert x["delta_bias"] is None
    dt = torch.nn.functional.softplus(x["delta"].double())
    # bf16 rounding of softplus^-1 moves the range ends a little
    assert dt.min() > 0.9e-3 and dt.max() < 1.1e-1
    lg = torch.log(dt)
    assert abs(lg.mean().item() - 0.5 * (math.log(1e-3) + math.log(1e-1))) < 0.05


def test_dna_recipe():
    w = small("dna1m", seqlen=4096, dim=32)
    x = W.scan_inputs(w)
    u = x["u"].float()[0]                         # [D, L]
    # every column is one of 4 embedding vectors plus N(0, 0.1) noise
    emb = u.t().numpy()
    d = ((emb[:, None, :] - emb[None, :64, :]) ** 2).mean(-1)    # distances to the first 64 columns
    close = d < 0.1
    assert close.sum(1).min() >= 1                 # every column has a near twin among the first 64
    assert u.std() > 0.5


def test_deterministic():
    w = small("mamba130m", batch=1, dim=8, seqlen=64)
    a, b = W.scan_inputs(w), W.scan_inputs(w)
    for k in ("u", "delta", "z", "B", "C", "delta_bias"):
        assert torch.equal(a[k], b[k])
    s0, s1 = W.decode_inputs(W.WORKLOADS["decode2p8b"].with_shape(batch=2, dim=16), 0), \
        W.decode_inputs(W.WORKLOADS["decode2p8b"].with_shape(batch=2, dim=16), 1)
    assert not torch.equal(s0["u"], s1["u"]) and s0["B"].shape == (2, 16)
