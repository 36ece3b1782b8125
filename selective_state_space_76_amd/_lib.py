"""ctypes binding of libssmscan.so (see include/ssm_scan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels of the
library.  There is no fallback: if the library is missing or no GPU is visible,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssmscan.so")

SSM_F32 = 0
SSM_BF16 = 1
SSM_FLAG_ZOH = 1
SSM_FLAG_REVERSE = 2
ABI_VERSION = 2

_STATUS = {0: "SSM_OK", 1: "SSM_ERR_NULL", 2: "SSM_ERR_SHAPE", 3: "SSM_ERR_DTYPE", 4: "SSM_ERR_ALIGN",
           5: "SSM_ERR_UNSUPPORTED", 6: "SSM_ERR_WORKSPACE", 7: "SSM_ERR_LAUNCH", 8: "SSM_ERR_OVERLAP",
           9: "SSM_ERR_TOO_LARGE"}


class SSMError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (_STATUS.get(status, "?"), status, message))
        self.status = status


class ssm_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


_lib = None
EXPORTS = ("ssm_abi_version", "ssm_status_str", "ssm_scan_workspace_size", "ssm_scan_fwd", "ssm_scan_fwd_save",
           "ssm_scan_fwd_noalloc",
           "ssm_state_update", "ssm_scan_bwd_workspace_size", "ssm_scan_bwd", "ssm_scan_bwd_saved_workspace_size",
           "ssm_scan_bwd_saved", "ssm_conv1d_fwd", "ssm_conv1d_update")


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libssmscan.so not found at %s; build it with "
                          "`python -m selective_state_space_76_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    lib.ssm_abi_version.argtypes = []
    lib.ssm_abi_version.restype = ctypes.c_int
    lib.ssm_status_str.argtypes = [ctypes.c_int]
    lib.ssm_status_str.restype = ctypes.c_char_p
    lib.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(ssm_shape)]
    lib.ssm_scan_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_fwd.argtypes = [ctypes.POINTER(ssm_shape)] + [vp] * 11 + [vp, ctypes.c_size_t, vp]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_save.argtypes = [ctypes.POINTER(ssm_shape)] + [vp] * 12 + [vp, ctypes.c_size_t, vp]
    lib.ssm_scan_fwd_save.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ssm_shape)] + [vp] * 11 + [vp]
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_state_update.argtypes = [i64, i64, i64, i32, u32] + [vp] * 10 + [vp]
    lib.ssm_state_update.restype = ctypes.c_int
    lib.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ssm_shape)]
    lib.ssm_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_bwd.argtypes = [ctypes.POINTER(ssm_shape)] + [vp] * 21 + [ctypes.c_size_t, vp]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_bwd_saved_workspace_size.argtypes = [ctypes.POINTER(ssm_shape)]
    lib.ssm_scan_bwd_saved_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_bwd_saved.argtypes = [ctypes.POINTER(ssm_shape)] + [vp] * 22 + [ctypes.c_size_t, vp]
    lib.ssm_scan_bwd_saved.restype = ctypes.c_int
    lib.ssm_conv1d_fwd.argtypes = [i64, i64, i64, i64, i32] + [vp] * 6 + [vp]
    lib.ssm_conv1d_fwd.restype = ctypes.c_int
    lib.ssm_conv1d_update.argtypes = [i64, i64, i64, i32] + [vp] * 5 + [vp]
    lib.ssm_conv1d_update.restype = ctypes.c_int
    if lib.ssm_abi_version() != ABI_VERSION:
        raise ImportError("libssmscan.so ABI version %d, binding expects %d" % (lib.ssm_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise SSMError(status, load().ssm_status_str(status).decode())


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("streams must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a tensor, got %r" % type(t))
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, shape, dtype, name, device=None):
    """The C ABI trusts sizes, element types and the device; check them here so a mismatched
    tensor is an error, not an out-of-bounds read."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s: expected a tensor on %s, got %s" % (name, device, t.device))


def _nonempty(**sizes):
    """The library computes nothing for an empty tensor and refuses one (SSM_ERR_SHAPE); say so
    here, by name, rather than pass on an empty tensor's null data pointer."""
    bad = ", ".join("%s=%d" % kv for kv in sizes.items() if kv[1] < 1)
    if bad:
        raise ValueError("empty input: every size must be at least 1 (%s)" % bad)


def _stream(stream, device):
    """The caller's stream, by default the current stream of the tensors' device."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(stream, *tensors):
    """Tensors this module allocated are taken from torch's current stream; when the kernels run
    on another stream, tell the caching allocator so the memory is not handed out again before
    that stream's work on it is done."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def make_shape(batch, dim, dstate, seqlen, io_dtype, zoh=False, reverse=False) -> ssm_shape:
    flags = (SSM_FLAG_ZOH if zoh else 0) | (SSM_FLAG_REVERSE if reverse else 0)
    return ssm_shape(int(batch), int(dim), int(dstate), int(seqlen), int(io_dtype), flags)


def workspace_size(batch, dim, dstate, seqlen, io_dtype=SSM_BF16, zoh=False, reverse=False) -> int:
    sh = make_shape(batch, dim, dstate, seqlen, io_dtype, zoh, reverse)
    return int(load().ssm_scan_workspace_size(ctypes.byref(sh)))


def checkpoints_shape(batch, dim, dstate, seqlen):
    """Shape of the block checkpoints scan_fwd(checkpoints=...) writes and scan_bwd reads."""
    return (batch, (seqlen + 63) // 64, dim, dstate)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, initial_state=None, *,
             out=None, final_state=True, zoh=False, reverse=False, workspace=None, split=True,
             checkpoints=None, stream=None):
    """Selective scan.  u, delta, z: [B,D,L]; B, C: [B,N,L] (same dtype as u); A: [D,N] fp32;
    D, delta_bias: [D] fp32; initial_state: [B,D,N] fp32 or None.
    Returns (out [B,D,L] in u's dtype, final_state [B,D,N] fp32 or None).
    final_state may be True (allocate), False/None (not written) or a tensor to write into.
    workspace: a uint8 tensor of at least workspace_size(...) bytes, or None to allocate one;
    split=False runs without a workspace (no sequence split).
    checkpoints: an fp32 tensor of checkpoints_shape(...) to also write the state entering every
    64-step block (ssm_scan_fwd_save), for scan_bwd(checkpoints=...)."""
    lib = load()
    Bsz, Dm, L = u.shape
    N = A.shape[1]
    _nonempty(batch=Bsz, dim=Dm, dstate=N, seqlen=L)
    io = _io_dtype(u)
    device = u.device
    sh = make_shape(Bsz, Dm, N, L, io, zoh, reverse)
    made = []  # tensors allocated here (on torch's current stream)
    if out is None:
        out = torch.empty_like(u)
        made.append(out)
    if final_state is True:
        final_state = torch.empty((Bsz, Dm, N), dtype=torch.float32, device=u.device)
        made.append(final_state)
    elif final_state is False:
        final_state = None
    f32 = torch.float32
    for t, shp, dt, name in ((delta, (Bsz, Dm, L), u.dtype, "delta"), (A, (Dm, N), f32, "A"),
                             (B, (Bsz, N, L), u.dtype, "B"), (C, (Bsz, N, L), u.dtype, "C"),
                             (D, (Dm,), f32, "D"), (z, (Bsz, Dm, L), u.dtype, "z"),
                             (delta_bias, (Dm,), f32, "delta_bias"),
                             (initial_state, (Bsz, Dm, N), f32, "initial_state"),
                             (out, (Bsz, Dm, L), u.dtype, "out"),
                             (final_state, (Bsz, Dm, N), f32, "final_state"),
                             (checkpoints, checkpoints_shape(Bsz, Dm, N, L), f32, "checkpoints")):
        _expect(t, shp, dt, name, device)
    ws_bytes = 0
    if workspace is not None and workspace.device != device:
        raise ValueError("workspace: expected a tensor on %s, got %s" % (device, workspace.device))
    if split:
        need = int(lib.ssm_scan_workspace_size(ctypes.byref(sh)))
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
            made.append(workspace)
        if workspace is not None:
            ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    if checkpoints is None:
        _check(lib.ssm_scan_fwd(ctypes.byref(sh), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(z), _ptr(delta_bias), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                _ptr(workspace), ws_bytes, _stream(stream, device)))
    else:
        _check(lib.ssm_scan_fwd_save(ctypes.byref(sh), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                     _ptr(z), _ptr(delta_bias), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                     _ptr(checkpoints), _ptr(workspace), ws_bytes, _stream(stream, device)))
    _on_stream(stream, *made)
    return out, final_state


SCRATCH_BYTES = 34 << 20  # the static scratch array behind ssm_scan_fwd_noalloc


def scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, initial_state=None, *, out, final_state=None,
                     zoh=False, reverse=False, stream=None):
    """ssm_scan_fwd_noalloc: the selective scan without a workspace; the library's static 34 MiB
    per-device scratch array holds a split sequence's segment summaries, and the call allocates
    nothing.  out (and final_state, if given) are the caller's tensors; arguments as scan_fwd.
    Calls that overlap in time on one GPU race on the shared scratch."""
    lib = load()
    Bsz, Dm, L = u.shape
    N = A.shape[1]
    _nonempty(batch=Bsz, dim=Dm, dstate=N, seqlen=L)
    io = _io_dtype(u)
    device = u.device
    sh = make_shape(Bsz, Dm, N, L, io, zoh, reverse)
    f32 = torch.float32
    for t, shp, dt, name in ((delta, (Bsz, Dm, L), u.dtype, "delta"), (A, (Dm, N), f32, "A"),
                             (B, (Bsz, N, L), u.dtype, "B"), (C, (Bsz, N, L), u.dtype, "C"),
                             (D, (Dm,), f32, "D"), (z, (Bsz, Dm, L), u.dtype, "z"),
                             (delta_bias, (Dm,), f32, "delta_bias"),
                             (initial_state, (Bsz, Dm, N), f32, "initial_state"),
                             (out, (Bsz, Dm, L), u.dtype, "out"),
                             (final_state, (Bsz, Dm, N), f32, "final_state")):
        _expect(t, shp, dt, name, device)
    _check(lib.ssm_scan_fwd_noalloc(ctypes.byref(sh), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(z), _ptr(delta_bias), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                    _stream(stream, device)))
    return out, final_state


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, *, out=None, zoh=False,
                 stream=None):
    """One recurrent step, state [B,D,N] fp32 updated in place.  u, delta, z: [B,D]; B, C: [B,N].
    Returns out [B,D] in u's dtype."""
    lib = load()
    Bsz, Dm = u.shape
    N = A.shape[1]
    _nonempty(batch=Bsz, dim=Dm, dstate=N)
    io = _io_dtype(u)
    device = u.device
    made = []
    if out is None:
        out = torch.empty_like(u)
        made.append(out)
    f32 = torch.float32
    for t, shp, dt, name in ((state, (Bsz, Dm, N), f32, "state"), (delta, (Bsz, Dm), u.dtype, "delta"),
                             (A, (Dm, N), f32, "A"), (B, (Bsz, N), u.dtype, "B"), (C, (Bsz, N), u.dtype, "C"),
                             (D, (Dm,), f32, "D"), (z, (Bsz, Dm), u.dtype, "z"),
                             (delta_bias, (Dm,), f32, "delta_bias"), (out, (Bsz, Dm), u.dtype, "out")):
        _expect(t, shp, dt, name, device)
    _check(lib.ssm_state_update(Bsz, Dm, N, io, SSM_FLAG_ZOH if zoh else 0, _ptr(state), _ptr(u), _ptr(delta),
                                _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(out),
                                _stream(stream, device)))
    _on_stream(stream, *made)
    return out


def bwd_workspace_size(batch, dim, dstate, seqlen, io_dtype=SSM_BF16, reverse=False, saved=False) -> int:
    """Workspace bytes of scan_bwd; saved=True: with the forward's checkpoints given."""
    sh = make_shape(batch, dim, dstate, seqlen, io_dtype, False, reverse)
    fn = load().ssm_scan_bwd_saved_workspace_size if saved else load().ssm_scan_bwd_workspace_size
    return int(fn(ctypes.byref(sh)))


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, initial_state=None, *, dout,
             dfinal_state=None, zoh=False, reverse=False, grads=None, workspace=None, checkpoints=None,
             stream=None):
    """Gradients of scan_fwd for output gradient dout [B,D,L] (u's dtype) and optional
    final-state gradient [B,D,N] fp32.  Returns a dict: du, ddelta (u's dtype), dA [D,N], dB, dC
    [B,N,L], dD, ddelta_bias [D] (fp32), dz (u's dtype, None without z) and dinitial_state
    [B,D,N] fp32.  grads: optional dict of preallocated outputs with those names.
    checkpoints: the tensor scan_fwd(checkpoints=...) wrote for the same inputs; the backward
    then skips its own checkpoint pass (ssm_scan_bwd_saved)."""
    lib = load()
    Bsz, Dm, L = u.shape
    N = A.shape[1]
    _nonempty(batch=Bsz, dim=Dm, dstate=N, seqlen=L)
    io = _io_dtype(u)
    device = u.device
    sh = make_shape(Bsz, Dm, N, L, io, zoh, reverse)
    f32, dev = torch.float32, u.device
    for t, shp, dt, name in ((delta, (Bsz, Dm, L), u.dtype, "delta"), (A, (Dm, N), f32, "A"),
                             (B, (Bsz, N, L), u.dtype, "B"), (C, (Bsz, N, L), u.dtype, "C"),
                             (D, (Dm,), f32, "D"), (z, (Bsz, Dm, L), u.dtype, "z"),
                             (delta_bias, (Dm,), f32, "delta_bias"),
                             (initial_state, (Bsz, Dm, N), f32, "initial_state"),
                             (dout, (Bsz, Dm, L), u.dtype, "dout"),
                             (dfinal_state, (Bsz, Dm, N), f32, "dfinal_state"),
                             (checkpoints, checkpoints_shape(Bsz, Dm, N, L), f32, "checkpoints")):
        _expect(t, shp, dt, name, device)
    shapes = dict(du=((Bsz, Dm, L), u.dtype), ddelta=((Bsz, Dm, L), u.dtype), dA=((Dm, N), f32),
                  dB=((Bsz, N, L), f32), dC=((Bsz, N, L), f32), dD=((Dm,), f32),
                  dz=((Bsz, Dm, L), u.dtype), ddelta_bias=((Dm,), f32), dinitial_state=((Bsz, Dm, N), f32))
    g = dict(grads or {})
    made = []
    for k, (shp, dt) in shapes.items():
        if k == "dz" and z is None:
            g[k] = None
            continue
        if g.get(k) is None:
            g[k] = torch.empty(shp, dtype=dt, device=dev)
            made.append(g[k])
        _expect(g[k], shp, dt, k, device)
    size_fn = lib.ssm_scan_bwd_workspace_size if checkpoints is None else lib.ssm_scan_bwd_saved_workspace_size
    need = int(size_fn(ctypes.byref(sh)))
    if workspace is not None and workspace.device != device:
        raise ValueError("workspace: expected a tensor on %s, got %s" % (device, workspace.device))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        made.append(workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    outs = (_ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
            _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dinitial_state"]))
    ins = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
           _ptr(initial_state), _ptr(dout), _ptr(dfinal_state))
    if checkpoints is None:
        _check(lib.ssm_scan_bwd(ctypes.byref(sh), *ins, *outs, _ptr(workspace), ws_bytes, _stream(stream, device)))
    else:
        _check(lib.ssm_scan_bwd_saved(ctypes.byref(sh), *ins, _ptr(checkpoints), *outs, _ptr(workspace), ws_bytes,
                                      _stream(stream, device)))
    _on_stream(stream, *made)
    return g


def conv1d_fwd(x, weight, bias=None, initial_state=None, *, out=None, final_state=True, stream=None):
    """Causal depthwise conv1d + bias + SiLU, producing u.  x: [B,D,L] fp32/bf16; weight: [D,K]
    fp32 (K in 1..4); bias: [D] fp32 or None; initial_state: [B,D,K-1] in x's dtype or None.
    Returns (u [B,D,L], final_state [B,D,K-1] or None).  final_state may be True (allocate),
    False/None (not written) or a tensor (not overlapping initial_state)."""
    lib = load()
    Bsz, Dm, L = x.shape
    K = weight.shape[1]
    _nonempty(batch=Bsz, dim=Dm, seqlen=L, width=K)
    io = _io_dtype(x)
    device = x.device
    made = []
    if out is None:
        out = torch.empty_like(x)
        made.append(out)
    if final_state is True:
        final_state = torch.empty((Bsz, Dm, K - 1), dtype=x.dtype, device=x.device)
        made.append(final_state)
    elif final_state is False:
        final_state = None
    f32 = torch.float32
    for t, shp, dt, name in ((weight, (Dm, K), f32, "weight"), (bias, (Dm,), f32, "bias"),
                             (initial_state, (Bsz, Dm, K - 1), x.dtype, "initial_state"),
                             (out, (Bsz, Dm, L), x.dtype, "out"),
                             (final_state, (Bsz, Dm, K - 1), x.dtype, "final_state")):
        _expect(t, shp, dt, name, device)
    _check(lib.ssm_conv1d_fwd(Bsz, Dm, L, K, io, _ptr(x), _ptr(weight), _ptr(bias), _ptr(initial_state),
                              _ptr(out), _ptr(final_state), _stream(stream, device)))
    _on_stream(stream, *made)
    return out, final_state


def conv1d_update(conv_state, x, weight, bias=None, *, out=None, stream=None):
    """One decode step of the conv: conv_state [B,D,K-1] (x's dtype) updated in place;
    x: [B,D].  Returns u [B,D]."""
    lib = load()
    Bsz, Dm = x.shape
    K = weight.shape[1]
    _nonempty(batch=Bsz, dim=Dm, width=K)
    io = _io_dtype(x)
    device = x.device
    made = []
    if out is None:
        out = torch.empty_like(x)
        made.append(out)
    f32 = torch.float32
    for t, shp, dt, name in ((conv_state, (Bsz, Dm, K - 1), x.dtype, "conv_state"),
                             (weight, (Dm, K), f32, "weight"), (bias, (Dm,), f32, "bias"),
                             (out, (Bsz, Dm), x.dtype, "out")):
        _expect(t, shp, dt, name, device)
    _check(lib.ssm_conv1d_update(Bsz, Dm, K, io, _ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias),
                                 _ptr(out), _stream(stream, device)))
    _on_stream(stream, *made)
    return out
