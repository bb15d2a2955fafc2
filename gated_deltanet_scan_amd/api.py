"""Torch-facing wrappers of the C ABI (argument marshalling only).

Every step of the scan runs in the HIP kernels of libgdn.so; this module only
checks tensor placement, allocates outputs and workspace with torch, and passes
raw device pointers plus torch's current HIP stream across the ABI.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import GdnDesc, GdnError


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def make_desc(B, H, F, N, D, dtype: torch.dtype, *, gates_are_logits=False, eps=1e-6) -> GdnDesc:
    if dtype == torch.bfloat16:
        io = _lib.GDN_BF16
    elif dtype == torch.float32:
        io = _lib.GDN_F32
    else:
        raise TypeError("q/k/v must be bfloat16 or float32")
    flags = _lib.GDN_FLAG_GATES_ARE_LOGITS if gates_are_logits else 0
    return GdnDesc(B, H, F, N, D, D, io, flags, float(eps))


def workspace_size(desc: GdnDesc) -> int:
    return int(_lib.load().gdn_workspace_size(ctypes.byref(desc)))


def alloc_workspace(desc: GdnDesc, device) -> Optional[torch.Tensor]:
    n = workspace_size(desc)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def _run(fn_name, q, k, v, beta, alpha, S_in, o, S_out, workspace, desc, stream):
    lib = _lib.load()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = getattr(lib, fn_name)(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                               _ptr(alpha), _ptr(S_in), _ptr(o), _ptr(S_out), _ptr(workspace),
                               ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, fn_name)


def frame_scan_fwd(q, k, v, beta, alpha, S0=None, *, gates_are_logits: bool = False,
                   eps: float = 1e-6, o=None, S_final=None, workspace=None,
                   return_state: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Whole-clip frame-wise GDN scan.

    q, k: [B,F,N,H,D]; v: [B,F,N,H,D] (bf16 or fp32, all the same dtype);
    beta: [B,F,N,H] fp32; alpha: [B,F,H] fp32; S0: [B,H,D,D] fp32 or None.
    Returns (o [B,F,N,H,D] in the q dtype, S_final [B,H,D,D] fp32 or None).
    """
    B, F, N, H, D = q.shape
    _check(q, "q", q.dtype, (B, F, N, H, D))
    _check(k, "k", q.dtype, (B, F, N, H, D))
    _check(v, "v", q.dtype, (B, F, N, H, D))
    _check(beta, "beta", torch.float32, (B, F, N, H))
    _check(alpha, "alpha", torch.float32, (B, F, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, (B, H, D, D))
    desc = make_desc(B, H, F, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps)
    if o is None:
        o = torch.empty_like(q)
    else:
        _check(o, "o", q.dtype, (B, F, N, H, D))
    if S_final is None and return_state:
        S_final = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    elif S_final is not None:
        _check(S_final, "S_final", torch.float32, (B, H, D, D))
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    _run("gdn_frame_scan_fwd", q, k, v, beta, alpha, S0, o, S_final, workspace, desc, stream)
    return o, S_final


def frame_step(q, k, v, beta, alpha, S_in=None, *, gates_are_logits: bool = False,
               eps: float = 1e-6, o=None, S_out=None, workspace=None, stream=None):
    """One frame of the scan for streaming use.

    q, k, v: [B,N,H,D] (or [B,1,N,H,D]); beta: [B,N,H] (or [B,1,N,H]);
    alpha: [B,H] (or [B,1,H]); S_in: [B,H,D,D] fp32 or None (zeros).
    S_out may be S_in itself (in-place carry).  Returns (o, S_out).
    """
    squeeze = q.dim() == 4
    if squeeze:
        q, k, v = q.unsqueeze(1), k.unsqueeze(1), v.unsqueeze(1)
        beta, alpha = beta.unsqueeze(1), alpha.unsqueeze(1)
        if o is not None:
            o = o.unsqueeze(1)
    B, F, N, H, D = q.shape
    if F != 1:
        raise ValueError("frame_step takes exactly one frame")
    _check(q, "q", q.dtype, (B, 1, N, H, D))
    _check(k, "k", q.dtype, (B, 1, N, H, D))
    _check(v, "v", q.dtype, (B, 1, N, H, D))
    _check(beta, "beta", torch.float32, (B, 1, N, H))
    _check(alpha, "alpha", torch.float32, (B, 1, H))
    if S_in is not None:
        _check(S_in, "S_in", torch.float32, (B, H, D, D))
    desc = make_desc(B, H, 1, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps)
    if o is None:
        o = torch.empty_like(q)
    if S_out is None:
        S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _check(S_out, "S_out", torch.float32, (B, H, D, D))
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    _run("gdn_frame_step", q, k, v, beta, alpha, S_in, o, S_out, workspace, desc, stream)
    return (o.squeeze(1) if squeeze else o), S_out


def profile_begin() -> None:
    st = _lib.load().gdn_profile_begin()
    if st != 0:
        raise GdnError(st, "gdn_profile_begin")


def profile_end() -> dict:
    """Stop profiling; {kernel name: (total ms, launches)} for every kernel kind."""
    lib = _lib.load()
    ms = (ctypes.c_double * _lib.GDN_NUM_KERNELS)()
    n = (ctypes.c_int64 * _lib.GDN_NUM_KERNELS)()
    st = lib.gdn_profile_end(ms, n)
    if st != 0:
        raise GdnError(st, "gdn_profile_end")
    return {lib.gdn_kernel_name(i).decode(): (ms[i], int(n[i])) for i in range(_lib.GDN_NUM_KERNELS)}
