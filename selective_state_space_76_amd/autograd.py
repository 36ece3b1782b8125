"""torch.autograd binding of the scan: forward through ssm_scan_fwd_save (the outputs plus the block
checkpoints), backward through ssm_scan_bwd_saved.

    from selective_state_space_76_amd import selective_scan
    out, last_state = selective_scan(u, delta, A, B, C, D, z, delta_bias)
    loss(out).backward()          # gradients of u, delta, A, B, C, D, z, delta_bias, initial_state

Bookkeeping only: the forward and backward arithmetic both run in the library's HIP kernels (the
gradients are the chain rule applied to the pages' forward recurrence, see include/ssm_scan.h).
Gradients are returned in each input's dtype; the library computes dA, dB, dC, dD and d(delta_bias)
in fp32 and they are cast to bf16 when those inputs are bf16.  Both discretisations (the default
dt*B and zero-order hold) and both scan directions have gradients.
"""
from __future__ import annotations

import torch

from ._lib import checkpoints_shape, scan_bwd, scan_fwd


class SelectiveScanFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, initial_state, zoh, reverse):
        # when a gradient will be asked for, the forward also writes the state entering every
        # 64-step block, and the backward starts from them instead of recomputing them
        ck = None
        if any(ctx.needs_input_grad[:9]):
            Bsz, Dm, L = u.shape
            ck = torch.empty(checkpoints_shape(Bsz, Dm, A.shape[1], L), dtype=torch.float32, device=u.device)
        out, final_state = scan_fwd(u, delta, A, B, C, D, z, delta_bias, initial_state, zoh=zoh, reverse=reverse,
                                    checkpoints=ck)
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, initial_state, ck)
        ctx.zoh, ctx.reverse = zoh, reverse
        return out, final_state

    @staticmethod
    def backward(ctx, dout, dfinal):
        u, delta, A, B, C, D, z, delta_bias, initial_state, ck = ctx.saved_tensors
        dout = torch.zeros_like(u) if dout is None else dout.to(u.dtype).contiguous()
        dfinal = None if dfinal is None else dfinal.float().contiguous()
        g = scan_bwd(u, delta, A, B, C, D, z, delta_bias, initial_state, dout=dout, dfinal_state=dfinal,
                     zoh=ctx.zoh, reverse=ctx.reverse, checkpoints=ck)
        need = ctx.needs_input_grad

        def cast(grad, like, i):
            return grad.to(like.dtype) if (need[i] and grad is not None and like is not None) else None

        return (cast(g["du"], u, 0), cast(g["ddelta"], delta, 1), cast(g["dA"], A, 2), cast(g["dB"], B, 3),
                cast(g["dC"], C, 4), cast(g["dD"], D, 5), cast(g["dz"], z, 6), cast(g["ddelta_bias"], delta_bias, 7),
                cast(g["dinitial_state"], initial_state, 8), None, None)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, initial_state=None, *, zoh=False,
                   reverse=False):
    """Differentiable selective scan.  Same arguments and layouts as scan_fwd; returns
    (out [B,D,L] in u's dtype, final_state [B,D,N] fp32)."""
    return SelectiveScanFn.apply(u, delta, A, B, C, D, z, delta_bias, initial_state, zoh, reverse)
