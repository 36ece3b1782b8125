"""fp64 CPU oracle for the selective state-space scan -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library and is never used
as a fallback for it.  The arithmetic lives in ``ssm_oracle.c`` (plain C,
double precision, OpenMP over independent channels); this module only builds
that file with gcc, widens inputs exactly to float64 and calls it.

What it computes follows the pages' definition of the selective SSM:
  * softplus step size with a per-channel bias inside (freeguideonline.com
    Mamba tutorial, section 4.2, step 2);
  * A_bar = exp(dt*A), B_bar = dt*B, h = A_bar*h + B_bar*x, y = C.h + D*x
    (fsdata.site "mamba-state-space-model" article, section 3.2);
  * SiLU gate of the second branch (ai.xwebgame.com Mamba page, PyTorch
    section);
  * optional exact ZOH B_bar (freeguideonline tutorial, section 2.2), reverse
    direction (fsdata.site article, section 7 pitfalls table) and a given
    initial state (mlqm.cn article, section 6.2, chunked long sequences);
  * the step that produces u: causal depthwise conv1d of width K with a bias,
    cut to the sequence length, then SiLU (ai.xwebgame.com Mamba page, the
    PyTorch block's step 2);
  * the gradients of the scan: not on the pages; the chain rule applied to the
    definition above, as a reverse-time adjoint recurrence (scan_bwd).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")

ZOH = 1
REVERSE = 2


def build(force: bool = False) -> str:
    """Compile ssm_oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """A loaded copy of the C oracle (the default one, or a variant built from edited source)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_scan_f64.argtypes = [i64, i64, i64, i64] + [d] * 11 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_scan_f64.restype = ctypes.c_int
        lib.oracle_step_f64.argtypes = [i64, i64, i64, d] + [d] * 8 + [d, ctypes.c_int, ctypes.c_int]
        lib.oracle_step_f64.restype = ctypes.c_int
        lib.oracle_conv1d_f64.argtypes = [i64, i64, i64, i64] + [d] * 6 + [ctypes.c_int]
        lib.oracle_conv1d_f64.restype = ctypes.c_int
        lib.oracle_scan_bwd_f64.argtypes = [i64, i64, i64, i64] + [d] * 20 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_scan_bwd_f64.restype = ctypes.c_int
        self.lib = lib

    def scan(self, u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None,
             zoh=False, reverse=False, threads=0):
        """Sequential fp64 selective scan.

        u, delta, z: [Bsz, Dm, L]; B, C: [Bsz, N, L]; A: [Dm, N]; D, delta_bias: [Dm];
        h0: [Bsz, Dm, N] or None (zero).  Returns (out [Bsz,Dm,L], final_state [Bsz,Dm,N]).
        """
        u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
        D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
        Bsz, Dm, L = u.shape
        N = A.shape[1]
        assert delta.shape == u.shape and A.shape == (Dm, N)
        assert B.shape == (Bsz, N, L) and C.shape == (Bsz, N, L)
        assert z is None or z.shape == u.shape
        assert D is None or D.shape == (Dm,)
        assert delta_bias is None or delta_bias.shape == (Dm,)
        assert h0 is None or h0.shape == (Bsz, Dm, N)
        out = np.empty((Bsz, Dm, L), np.float64)
        fs = np.empty((Bsz, Dm, N), np.float64)
        flags = (ZOH if zoh else 0) | (REVERSE if reverse else 0)
        rc = self.lib.oracle_scan_f64(Bsz, Dm, N, L, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                      _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(out),
                                      _ptr(fs), flags, int(threads))
        if rc != 0:
            raise RuntimeError("oracle_scan_f64 failed (%d)" % rc)
        return out, fs

    def step(self, state, u, delta, A, B, C, D=None, z=None, delta_bias=None, zoh=False, threads=0):
        """One fp64 recurrent update; `state` [Bsz,Dm,N] is not modified.  Returns (out [Bsz,Dm], new_state)."""
        st = _f64(state).copy()
        u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
        D, z, delta_bias = map(_f64, (D, z, delta_bias))
        Bsz, Dm = u.shape
        N = A.shape[1]
        assert st.shape == (Bsz, Dm, N) and B.shape == (Bsz, N) and C.shape == (Bsz, N)
        out = np.empty((Bsz, Dm), np.float64)
        rc = self.lib.oracle_step_f64(Bsz, Dm, N, _ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                      _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(out),
                                      ZOH if zoh else 0, int(threads))
        if rc != 0:
            raise RuntimeError("oracle_step_f64 failed (%d)" % rc)
        return out, st

    def scan_bwd(self, u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *, dout,
                 dfinal=None, zoh=False, reverse=False, threads=0):
        """Gradients of the scan for output gradient dout [Bsz,Dm,L] (and final-state gradient
        dfinal [Bsz,Dm,N] or None).  Returns a dict with du, ddelta, dA, dB, dC and, when the
        matching input is given, dD, dz, ddelta_bias, dh0 (dh0 always: the gradient of the
        state before the first step)."""
        u, delta, A, B, C, dout = map(_f64, (u, delta, A, B, C, dout))
        D, z, delta_bias, h0, dfinal = map(_f64, (D, z, delta_bias, h0, dfinal))
        Bsz, Dm, L = u.shape
        N = A.shape[1]
        assert delta.shape == u.shape and dout.shape == u.shape and A.shape == (Dm, N)
        assert B.shape == (Bsz, N, L) and C.shape == (Bsz, N, L)
        assert dfinal is None or dfinal.shape == (Bsz, Dm, N)
        g = dict(du=np.empty((Bsz, Dm, L)), ddelta=np.empty((Bsz, Dm, L)), dA=np.empty((Dm, N)),
                 dB=np.empty((Bsz, N, L)), dC=np.empty((Bsz, N, L)), dD=np.empty(Dm),
                 dz=np.empty((Bsz, Dm, L)) if z is not None else None, ddelta_bias=np.empty(Dm),
                 dh0=np.empty((Bsz, Dm, N)))
        rc = self.lib.oracle_scan_bwd_f64(
            Bsz, Dm, N, L, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), _ptr(h0), _ptr(dout), _ptr(dfinal), _ptr(g["du"]), _ptr(g["ddelta"]),
            _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
            _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), (ZOH if zoh else 0) | (REVERSE if reverse else 0),
            int(threads))
        if rc != 0:
            raise RuntimeError("oracle_scan_bwd_f64 failed (%d)" % rc)
        if D is None:
            g["dD"] = None
        if delta_bias is None:
            g["ddelta_bias"] = None
        if z is None:
            g["dz"] = None
        return g

    def conv1d(self, x, w, bias=None, state=None, threads=0):
        """Causal depthwise conv1d + bias + SiLU in fp64.

        x: [Bsz, Dm, L]; w: [Dm, K]; bias: [Dm] or None; state: [Bsz, Dm, K-1] inputs before
        x (oldest first) or None (zeros).  Returns (u [Bsz,Dm,L], state_out [Bsz,Dm,K-1]).
        """
        x, w, bias, state = map(_f64, (x, w, bias, state))
        Bsz, Dm, L = x.shape
        K = w.shape[1]
        assert w.shape == (Dm, K) and K >= 1
        assert bias is None or bias.shape == (Dm,)
        assert state is None or state.shape == (Bsz, Dm, K - 1)
        u = np.empty((Bsz, Dm, L), np.float64)
        so = np.empty((Bsz, Dm, K - 1), np.float64)
        rc = self.lib.oracle_conv1d_f64(Bsz, Dm, L, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(state),
                                        _ptr(u), _ptr(so), int(threads))
        if rc != 0:
            raise RuntimeError("oracle_conv1d_f64 failed (%d)" % rc)
        return u, so

    def conv_step(self, state, x, w, bias=None):
        """One decode step of the conv: the L = 1 case.  x: [Bsz, Dm]; state: [Bsz, Dm, K-1].
        Returns (u [Bsz, Dm], new_state [Bsz, Dm, K-1])."""
        x = _f64(x)
        u, so = self.conv1d(x[:, :, None], w, bias, state)
        return u[:, :, 0], so


def compile_variant(src_text: str, out_path: str) -> str:
    """Build an edited copy of the oracle source (used to check that the pins catch mistakes)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                           "-std=c11", "-w", "-o", out_path, src, "-lm"])
    return out_path


def source() -> str:
    with open(_SRC) as f:
        return f.read()


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def max_threads() -> int:
    """Threads the oracle's OpenMP loops use by default."""
    lib = default().lib
    lib.oracle_max_threads.restype = ctypes.c_int
    return int(lib.oracle_max_threads())


def scan(*args, **kw):
    return default().scan(*args, **kw)


def step(*args, **kw):
    return default().step(*args, **kw)


def conv1d(*args, **kw):
    return default().conv1d(*args, **kw)


def scan_bwd(*args, **kw):
    return default().scan_bwd(*args, **kw)


def conv_step(*args, **kw):
    return default().conv_step(*args, **kw)


def _f64(x):
    """Exact widening to a contiguous float64 array (bf16 and fp32 embed exactly)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
