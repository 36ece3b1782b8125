"""Decode steps and a training step captured in a HIP graph and replayed (GPU).

A serving loop issues the decode step's small kernels from a captured graph.  The
library launches only kernels on the caller's stream (no allocation, no memset),
so the calls can be captured.  Each replay runs after eager work that resets the
states and a synchronisation, and must reproduce the eager results bit for bit."""
import pytest
import torch

from selective_state_space_76_amd import (bwd_workspace_size, conv1d_fwd, conv1d_update, scan_bwd, scan_fwd,
                                          state_update, workspace_size)
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


@pytest.mark.parametrize("Bsz,Dm,N,L", [(2, 64, 16, 300), (1, 20, 16, 5000), (1, 20, 64, 4100), (1, 128, 16, 4096)],
                         ids=["whole", "split16", "split64", "split16_channels_on_lanes"])
def test_training_step_in_graph_matches_eager(Bsz, Dm, N, L):
    """conv1d + SiLU, the scan and its backward (with the sequence split where the shape asks
    for it) captured once and replayed: every output bit for bit equal to the eager call."""
    w = W.WORKLOADS["mamba130m"].with_shape(batch=Bsz, dim=Dm, dstate=N, seqlen=L, seed=5100 + N)
    K = 4
    x = W.scan_inputs(w, device=DEV)
    conv = W.conv_inputs(w, K, device=DEV)
    cw, cb = conv["weight"], conv["bias"]
    g = torch.Generator(device=DEV).manual_seed(5200)
    dout = torch.randn(Bsz, Dm, L, generator=g, device=DEV).to(torch.bfloat16)
    h0 = torch.randn(Bsz, Dm, N, generator=g, device=DEV)
    xin = conv["x"]
    u = torch.empty_like(xin)
    out = torch.empty_like(xin)
    fs = torch.empty(Bsz, Dm, N, device=DEV)
    fws = torch.empty(max(1, workspace_size(Bsz, Dm, N, L)), dtype=torch.uint8, device=DEV)
    bws = torch.empty(bwd_workspace_size(Bsz, Dm, N, L), dtype=torch.uint8, device=DEV)
    grads = {}

    def step():
        conv1d_fwd(xin, cw, cb, out=u, final_state=False)
        scan_fwd(u, x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], h0, out=out,
                 final_state=fs, workspace=fws)
        r = scan_bwd(u, x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], h0, dout=dout,
                     dfinal_state=fs, grads=grads or None, workspace=bws)
        grads.update(r)

    step()
    torch.cuda.synchronize()
    ref = {"u": u.clone(), "out": out.clone(), "fs": fs.clone()}
    ref.update({k: v.clone() for k, v in grads.items() if v is not None})

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        print("case: training-step graph %dx%dx%dx%d replay %d" % (Bsz, Dm, N, L, rep), flush=True)
        for t in [u, out, fs] + [v for v in grads.values() if v is not None]:
            t.zero_()           # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"u": u, "out": out, "fs": fs}
        got.update({k: v for k, v in grads.items() if v is not None})
        for k, v in ref.items():
            assert torch.equal(got[k], v), (rep, k)
