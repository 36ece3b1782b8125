"""MI355X (gfx950) selective state-space scan: HIP kernels behind a C ABI.

    from selective_state_space_76_amd import conv1d_fwd, scan_fwd, state_update, conv1d_update
    u, conv_state = conv1d_fwd(x, conv_weight, conv_bias)          # the step that produces u
    out, h_last = scan_fwd(u, delta, A, B, C, D, z, delta_bias)    # prefill
    grads = scan_bwd(u, delta, A, B, C, D, z, delta_bias, dout=g)  # training backward
    out, h_last = selective_scan(u, delta, A, B, C, D, z, delta_bias)  # the same, under autograd
    u_t = conv1d_update(conv_state, x_t, conv_weight, conv_bias)   # decode
    y = state_update(h_last, u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias)

The C ABI is include/ssm_scan.h; the library is libssmscan.so in this package,
built by `python -m selective_state_space_76_amd.build`.
"""
from ._lib import (SSMError, load, scan_fwd, scan_fwd_noalloc, state_update, conv1d_fwd, conv1d_update,  # noqa: F401
                   scan_bwd, bwd_workspace_size, workspace_size, checkpoints_shape, SSM_F32, SSM_BF16,
                   SSM_FLAG_ZOH, SSM_FLAG_REVERSE, LIB_PATH)
from .autograd import SelectiveScanFn, selective_scan  # noqa: F401

__all__ = ["scan_fwd", "scan_fwd_noalloc", "scan_bwd", "selective_scan", "SelectiveScanFn", "state_update", "conv1d_fwd",
           "conv1d_update", "workspace_size", "bwd_workspace_size", "checkpoints_shape", "load", "SSMError",
           "LIB_PATH"]
