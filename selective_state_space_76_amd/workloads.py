"""Seeded synthetic workloads for the selective scan (shapes + input recipes).

This module only draws inputs: it holds none of the scan's arithmetic, and both
the HIP path and the CPU oracle consume exactly the tensors it returns (the
oracle widens the same bf16/fp32 bits to float64).

Workloads (stand-ins for the pages' settings; their datasets are not used):
  tiny        1 x 64 channels x 16 states x 256 steps, all fp32 (parity case)
  mamba130m   8 x 1536 x 16 x 2048, bf16 streams -- a 130M-class layer
              (d_inner = 2 x 768, d_state 16)
  mamba1p3b   4 x 4096 x 64 x 4096, bf16 streams, no dt bias, step sizes drawn
              log-uniform directly -- a 1.3B-class layer with a wide state
  dna1m       1 x 1024 x 16 x 1,048,576, bf16 streams; u embeds i.i.d. 4-letter
              tokens -- the pages' million-base DNA sequences
  decode2p8b  256 x 5120 x 16, one token per step, fresh inputs every step --
              recurrent generation at a 2.8B-class width

Value recipe shared by all: u, z ~ N(0,1); delta ~ 0.5 N(0,1); per-channel
dt_bias = softplus^-1(Delta*), Delta* log-uniform in [1e-3, 1e-1];
A[d, n] = -(n + 1); B, C ~ N(0,1) per (batch, state, step), shared by channels;
D = 1.  bf16 tensors are drawn in fp32 and rounded once (round-to-nearest-even).

The conv step that produces u (conv_inputs / conv_decode_inputs) takes the
same shapes: its input x ~ N(0,1) [B,D,L]; weight [D,K] and bias [D] drawn
uniform in +-1/sqrt(K) (the default initialisation of a depthwise Conv1d of
width K, the layer of the pages' PyTorch block); the carried state, when one is
used, ~ N(0,1).

Random numbers come from torch generators seeded per (workload seed, tensor id,
step), on the device the tensors are created on.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int            # 1 for decode workloads
    io: str                # "f32" or "bf16": dtype of u, delta, B, C, z and out
    recipe: str            # "base", "logu_delta" or "dna"
    bias: bool             # whether a per-channel dt bias is passed
    seed: int
    steps: int = 0         # decode workloads: number of consecutive tokens

    @property
    def torch_dtype(self):
        return torch.float32 if self.io == "f32" else torch.bfloat16

    @property
    def updates(self) -> int:
        """State updates (batch * steps * channels * states) of one scan call or decode step."""
        return self.batch * self.seqlen * self.dim * self.dstate

    def with_shape(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 16, 256, "f32", "base", True, 76000),
    "mamba130m": Workload("mamba130m", 8, 1536, 16, 2048, "bf16", "base", True, 76001),
    "mamba1p3b": Workload("mamba1p3b", 4, 4096, 64, 4096, "bf16", "logu_delta", False, 76002),
    "dna1m": Workload("dna1m", 1, 1024, 16, 1 << 20, "bf16", "dna", True, 76003),
    "decode2p8b": Workload("decode2p8b", 256, 5120, 16, 1, "bf16", "base", True, 76004, steps=1000),
}

# tensor ids used to derive independent generator streams
_TID = {"u": 1, "delta": 2, "z": 3, "B": 4, "C": 5, "bias": 6, "emb": 7, "tok": 8, "noise": 9,
        "cx": 10, "cw": 11, "cb": 12, "cst": 13}


def _gen(device, seed: int, tid: str, step: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + _TID[tid] * 7919 + step * 104729) % (2**63 - 1))
    return g


def _normal(shape, device, seed, tid, step=0, scale=1.0):
    x = torch.randn(shape, generator=_gen(device, seed, tid, step), device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x


def _inv_softplus(y: np.ndarray) -> np.ndarray:
    # inverse of log(1 + e^x): x = y + log(1 - e^-y)
    return y + np.log(-np.expm1(-y))


def _logu(n: int, rng: np.random.Generator) -> np.ndarray:
    return np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=n))


def params(w: Workload, device="cpu"):
    """Per-channel constants: A [D,N], D [D], dt_bias [D] (or None), all fp32."""
    A = -torch.arange(1, w.dstate + 1, dtype=torch.float32).repeat(w.dim, 1)
    Dv = torch.ones(w.dim, dtype=torch.float32)
    bias = None
    if w.bias:
        rng = np.random.default_rng(w.seed * 31 + _TID["bias"])
        bias = torch.from_numpy(_inv_softplus(_logu(w.dim, rng)).astype(np.float32))
        bias = bias.to(device)
    return A.to(device), Dv.to(device), bias


def scan_inputs(w: Workload, device="cpu"):
    """Inputs of one scan call: dict with u, delta, z [B,D,L]; B, C [B,N,L]; A, D, delta_bias."""
    dt = w.torch_dtype
    Bsz, Dm, N, L = w.batch, w.dim, w.dstate, w.seqlen
    shp = (Bsz, Dm, L)
    if w.recipe == "dna":
        emb = _normal((4, Dm), device, w.seed, "emb")
        tok = torch.randint(0, 4, (Bsz, L), generator=_gen(device, w.seed, "tok"), device=device)
        u = torch.empty(shp, dtype=dt, device=device)
        for b in range(Bsz):  # [L, D] -> [D, L], one batch row at a time to bound memory
            row = emb[tok[b]].t()
            row = row + _normal((Dm, L), device, w.seed, "noise", step=b, scale=0.1)
            u[b] = row.to(dt)
            del row
    else:
        u = _normal(shp, device, w.seed, "u").to(dt)
    if w.recipe == "logu_delta":
        g = _gen(device, w.seed, "delta")
        r = torch.rand(shp, generator=g, device=device, dtype=torch.float64)
        dstar = torch.exp(math.log(1e-3) + r * (math.log(1e-1) - math.log(1e-3)))
        delta = (dstar + torch.log(-torch.expm1(-dstar))).to(dt)
        del r, dstar
    else:
        delta = _normal(shp, device, w.seed, "delta", scale=0.5).to(dt)
    z = _normal(shp, device, w.seed, "z").to(dt)
    Bm = _normal((Bsz, N, L), device, w.seed, "B").to(dt)
    Cm = _normal((Bsz, N, L), device, w.seed, "C").to(dt)
    A, Dv, bias = params(w, device)
    return dict(u=u, delta=delta, A=A, B=Bm, C=Cm, D=Dv, z=z, delta_bias=bias)


def decode_inputs(w: Workload, step: int, device="cpu"):
    """Per-token inputs of decode step `step`: u, delta, z [B,D]; B, C [B,N]."""
    dt = w.torch_dtype
    shp = (w.batch, w.dim)
    return dict(
        u=_normal(shp, device, w.seed, "u", step).to(dt),
        delta=_normal(shp, device, w.seed, "delta", step, scale=0.5).to(dt),
        z=_normal(shp, device, w.seed, "z", step).to(dt),
        B=_normal((w.batch, w.dstate), device, w.seed, "B", step).to(dt),
        C=_normal((w.batch, w.dstate), device, w.seed, "C", step).to(dt),
    )


def _uniform(shape, device, seed, tid, bound, step=0):
    g = _gen(device, seed, tid, step)
    return (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0) * bound


def conv_params(w: Workload, width: int = 4, device="cpu"):
    """Conv weight [D, width] and bias [D], fp32, uniform in +-1/sqrt(width)."""
    bound = 1.0 / math.sqrt(width)
    return (_uniform((w.dim, width), device, w.seed, "cw", bound),
            _uniform((w.dim,), device, w.seed, "cb", bound))


def conv_inputs(w: Workload, width: int = 4, device="cpu", state: bool = False):
    """Inputs of one conv call: dict with x [B,D,L] (io dtype), weight, bias and, if asked,
    state [B,D,width-1] (io dtype)."""
    dt = w.torch_dtype
    x = _normal((w.batch, w.dim, w.seqlen), device, w.seed, "cx").to(dt)
    weight, bias = conv_params(w, width, device)
    out = dict(x=x, weight=weight, bias=bias)
    if state:
        out["state"] = _normal((w.batch, w.dim, width - 1), device, w.seed, "cst").to(dt)
    return out


def conv_decode_inputs(w: Workload, step: int, device="cpu"):
    """Per-token conv input x [B,D] of decode step `step`."""
    return _normal((w.batch, w.dim), device, w.seed, "cx", step).to(w.torch_dtype)
