"""Build libssmscan.so (gfx950) in-tree with hipcc.

    python -m selective_state_space_76_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssmscan.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "scan_bf16_out.hip", "scan_bf16_sum.hip", "scan_f32_out.hip", "scan_f32_sum.hip",
    "scan_cl.hip", "ssm_kernels.hip", "conv_kernels.hip", "scan_bwd.hip", "scan_bwd_zoh.hip", "ssm_abi.cpp")]
HEADERS = [os.path.join(CSRC, "ssm_launch.h"), os.path.join(CSRC, "ssm_device.h"),
           os.path.join(CSRC, "scan_bwd_kernel.h"),
           os.path.join(ROOT, "include", "ssm_scan.h")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # no packed fp32 instructions: plain scalar VALU fp32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile_cmd(src: str, obj: str):
    if src.endswith(".cpp"):
        flags = [f for f in HIPCC_FLAGS if not f.startswith("--offload-arch")]
        inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
        return [hipcc()] + flags + ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I" + inc, "-c", src, "-o", obj]
    return [hipcc()] + HIPCC_FLAGS + ["-c", src, "-o", obj]


PROBE_SRC = os.path.join(CSRC, "issue_probe.hip")
PROBE_LIB = os.path.join(PKG, "libssmprobe.so")
TP_SRC = os.path.join(CSRC, "scan_time_parallel.hip")
TP_LIB = os.path.join(PKG, "libssmtp.so")


def build_probe(verbose: bool = False) -> str:
    """The VALU issue-rate probe bench.py reports beside the scan (a separate library, not the ABI)."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-shared", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), r.stdout))
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build_tp(verbose: bool = False) -> str:
    """The scan in the time-parallel layout, which bench.py times beside the library's (a separate
    library, not the ABI)."""
    tmp = TP_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-shared", TP_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), r.stdout))
    os.replace(tmp, TP_LIB)
    return TP_LIB


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP/C++ source of the library (in parallel) and link libssmscan.so."""
    from concurrent.futures import ThreadPoolExecutor

    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    objs = [os.path.join(CSRC, os.path.basename(s) + ".o") for s in SOURCES]

    def one(pair):
        src, obj = pair
        cmd = _compile_cmd(src, obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), r.stdout))
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(one, zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
    print(build_tp(verbose="-v" in sys.argv))
