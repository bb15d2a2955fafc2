"""torch.autograd binding of the frame scan (argument marshalling only).

``frame_scan(q, k, v, beta, alpha, S0=None, ...)`` returns (o, S_final) as a
differentiable function of every tensor input: the forward pass is
gdn_frame_scan_fwd_save, which keeps each frame's operands for the backward
pass (gdn_saved_size bytes, held by the autograd graph until backward runs or
the graph is freed), and the backward pass is gdn_frame_scan_bwd_saved.  With
``recompute=True`` the forward pass keeps nothing and the backward pass
(gdn_frame_scan_bwd) recomputes the operands instead.  Both give the same
gradients bit for bit.
"""
from __future__ import annotations

import torch

from . import api


class _FrameScan(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, beta, alpha, S0, gates_are_logits, eps, normalize_keys, reverse, recompute):
        kw = dict(gates_are_logits=gates_are_logits, eps=eps, normalize_keys=normalize_keys, reverse=reverse)
        if recompute:
            o, S_final = api.frame_scan_fwd(q, k, v, beta, alpha, S0, **kw)
            saved = None
        else:
            o, S_final, saved = api.frame_scan_fwd_save(q, k, v, beta, alpha, S0, **kw)
        ctx.kw = kw
        ctx.has_S0 = S0 is not None
        ctx.saved_buf = saved
        # S0 is needed by the recomputing backward only (the saved buffer holds its copy)
        ctx.save_for_backward(q, k, v, beta, alpha, S0 if (recompute and S0 is not None) else None)
        return o, S_final

    @staticmethod
    def backward(ctx, dO, dS_final):
        q, k, v, beta, alpha, S0 = ctx.saved_tensors
        dO = torch.zeros_like(q) if dO is None else dO.contiguous().to(q.dtype)
        dS_final = None if dS_final is None else dS_final.contiguous().float()
        dq, dk, dv, dbeta, dalpha, dS0 = api.frame_scan_bwd(q, k, v, beta, alpha, dO, S0, dS_final,
                                                            return_dS0=ctx.has_S0, saved=ctx.saved_buf, **ctx.kw)
        ctx.saved_buf = None
        return dq, dk, dv, dbeta, dalpha, dS0, None, None, None, None, None


def frame_scan(q, k, v, beta, alpha, S0=None, *, gates_are_logits: bool = False, eps: float = 1e-6,
               normalize_keys: bool = True, reverse: bool = False, recompute: bool = False):
    """Differentiable whole-clip scan: (o, S_final) with gradients to q, k, v,
    beta, alpha and S0 (layouts as for api.frame_scan_fwd)."""
    return _FrameScan.apply(q, k, v, beta, alpha, S0, gates_are_logits, eps, normalize_keys, reverse, recompute)
