"""MI355X (gfx950) selective state-space scan: HIP kernels behind a C ABI.

    from selective_state_space_76_amd import scan_fwd, state_update
    out, h_last = scan_fwd(u, delta, A, B, C, D, z, delta_bias)
    y = state_update(state, u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias)

The C ABI is include/ssm_scan.h; the library is libssmscan.so in this package,
built by `python -m selective_state_space_76_amd.build`.
"""
from ._lib import (SSMError, load, scan_fwd, state_update, workspace_size, SSM_F32, SSM_BF16,  # noqa: F401
                   SSM_FLAG_ZOH, SSM_FLAG_REVERSE, LIB_PATH)

__all__ = ["scan_fwd", "state_update", "workspace_size", "load", "SSMError", "LIB_PATH"]
