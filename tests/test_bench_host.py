"""bench.py's host-side contract, on the CPU: the algorithmic byte counts its rooflines divide by,
the refusal of more than one GPU, and the counter files its `traffic` fields come from."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from selective_state_space_76_amd import workloads as W  # noqa: E402


def test_scan_bytes_by_hand():
    # (3 streams in + 1 out) x s x B D L + 2 x s x B N L (B, C) + A + D (+ bias) + final state
    w = W.WORKLOADS["mamba130m"]  # 8 x 1536 x 16 x 2048, bf16, with bias
    bdl, bnl = 8 * 1536 * 2048, 8 * 16 * 2048
    want = 4 * 2 * bdl + 2 * 2 * bnl + 4 * 1536 * 16 + 4 * 1536 * 2 + 4 * 8 * 1536 * 16
    assert bench.scan_bytes(w) == want == 203_272_192
    w = W.WORKLOADS["mamba1p3b"]  # 4 x 4096 x 64 x 4096, no bias
    bdl, bnl = 4 * 4096 * 4096, 4 * 64 * 4096
    assert bench.scan_bytes(w) == 4 * 2 * bdl + 2 * 2 * bnl + 4 * 4096 * 64 + 4 * 4096 + 4 * 4 * 4096 * 64
    assert bench.scan_bytes(W.WORKLOADS["dna1m"]) == 8_657_182_720


def test_step_and_conv_bytes_by_hand():
    w = W.WORKLOADS["decode2p8b"]  # 256 x 5120 x 16, bf16 per-token streams, fp32 state
    bd, bdn = 256 * 5120, 256 * 5120 * 16
    want = 2 * 4 * bdn + 4 * 2 * bd + 2 * 2 * 256 * 16 + 4 * 5120 * 16 + 8 * 5120
    assert bench.step_bytes(w) == want == 178_642_944
    # conv prefill, K = 4: x read, u written, the carried-out state written, weights + bias read
    m = W.WORKLOADS["mamba130m"]
    assert bench.conv_bytes(m, 4) == 2 * 2 * 8 * 1536 * 2048 + 2 * 8 * 1536 * 3 + 4 * 1536 * 5 == 100_767_744
    assert bench.conv_step_bytes(w, 4) == 2 * 2 * bd * 3 + 2 * 2 * bd + 4 * 5120 * 5 == 21_073_920


def test_bwd_bytes_by_hand():
    w = W.WORKLOADS["mamba130m"]
    bdl, bnl = 8 * 1536 * 2048, 8 * 16 * 2048
    # u, delta, z, dout in; B, C in; du, ddelta, dz out; dB, dC out in fp32; dA and A; D, dD, bias, dbias
    want = 4 * 2 * bdl + 2 * 2 * bnl + 3 * 2 * bdl + 2 * 4 * bnl + 2 * 4 * 1536 * 16 + 4 * 4 * 1536
    assert bench.bwd_bytes(w) == want == 355_688_448


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", ["dna1m", "mamba130m", "mamba1p3b", "decode2p8b", "bwd_mamba130m", "bwd_mamba1p3b",
                                  "conv_mamba130m", "conv_update_decode2p8b"])
def test_counter_files_for_every_record(name, monkeypatch):
    """Every record's `traffic` has its counter summary; it is reported only for the kernel sources
    it was measured on."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % name)
    with open(path) as f:
        c = json.load(f)
    assert c["hbm_bytes_per_launch"] > 0 and c["algorithmic_bytes_per_launch"] > 0
    assert c["fetch_scale"] > 0 and c["write_scale"] > 0
    assert all("rocprofv3" in cmd for cmd in c["commands"])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: c["kernel_source_hash"])
    assert bench.traffic_from_profile(name, 1) == c["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.traffic_from_profile(name, 1) is None


def test_time_parallel_library_is_built_and_exports_its_entry():
    """The layout comparison's library: built beside the scan library (build() compiles it) and
    loadable without a GPU."""
    lib = bench.tp_library()
    assert lib is not None
    assert hasattr(lib, "ssm_tp_scan_fwd")
