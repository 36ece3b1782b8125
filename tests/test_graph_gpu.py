"""Decode steps captured in a HIP graph and replayed (GPU).

A serving loop issues the decode step's small kernels from a captured graph.  The
library launches only kernels on the caller's stream (no allocation, no memset),
so the calls can be captured.  Each replay runs after eager work that resets the
states and a synchronisation, and must reproduce the eager results bit for bit."""
import pytest
import torch

from selective_state_space_76_amd import conv1d_update, state_update
from selective_state_space_76_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_decode_steps_in_graph_match_eager():
    w = W.WORKLOADS["decode2p8b"].with_shape(batch=4, dim=256, seed=5000)
    T, K = 5, 4
    A, Dv, bias = W.params(w, device=DEV)
    cw, cb = W.conv_params(w, K, device=DEV)
    xs = [W.conv_decode_inputs(w, t, device=DEV) for t in range(T)]
    ins = [W.decode_inputs(w, t, device=DEV) for t in range(T)]
    h0 = torch.randn(w.batch, w.dim, w.dstate, device=DEV)
    c0 = W.conv_inputs(w, K, device=DEV, state=True)["state"]

    hs = torch.empty_like(h0)
    cs = torch.empty_like(c0)
    us = [torch.empty(w.batch, w.dim, dtype=torch.bfloat16, device=DEV) for _ in range(T)]
    ys = [torch.empty(w.batch, w.dim, dtype=torch.bfloat16, device=DEV) for _ in range(T)]

    def steps():
        for t in range(T):
            conv1d_update(cs, xs[t], cw, cb, out=us[t])
            i = ins[t]
            state_update(hs, us[t], i["delta"], A, i["B"], i["C"], Dv, i["z"], bias, out=ys[t])

    hs.copy_(h0)
    cs.copy_(c0)
    steps()
    torch.cuda.synchronize()
    ref_y = [y.clone() for y in ys]
    ref_h, ref_c = hs.clone(), cs.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        print("case: graph replay %d" % rep, flush=True)
        hs.copy_(h0)            # eager work between replays
        cs.copy_(c0)
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(ys[t], ref_y[t]), (rep, t)
        assert torch.equal(hs, ref_h) and torch.equal(cs, ref_c), rep
