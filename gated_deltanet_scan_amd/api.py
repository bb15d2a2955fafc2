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


def make_desc(B, H, F, N, D, dtype: torch.dtype, *, gates_are_logits=False, eps=1e-6,
              normalize_keys=True, reverse=False) -> GdnDesc:
    if dtype == torch.bfloat16:
        io = _lib.GDN_BF16
    elif dtype == torch.float32:
        io = _lib.GDN_F32
    elif dtype == torch.float8_e4m3fn:
        io = _lib.GDN_FP8_E4M3
    else:
        raise TypeError("q/k/v must be bfloat16, float32 or float8_e4m3fn")
    flags = _lib.GDN_FLAG_GATES_ARE_LOGITS if gates_are_logits else 0
    if not normalize_keys:
        flags |= _lib.GDN_FLAG_NO_KEY_NORM
    if reverse:
        flags |= _lib.GDN_FLAG_REVERSE
    return GdnDesc(B, H, F, N, D, D, io, flags, float(eps))


def workspace_size(desc: GdnDesc) -> int:
    return int(_lib.load().gdn_workspace_size(ctypes.byref(desc)))


def alloc_workspace(desc: GdnDesc, device) -> Optional[torch.Tensor]:
    n = workspace_size(desc)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def _check_workspace(workspace, device):
    if workspace is None:
        return
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != device:
        raise ValueError("workspace must be on %s (got %s)" % (device, workspace.device))
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")


def _run(fn_name, q, k, v, beta, alpha, S_in, o, S_out, workspace, desc, stream):
    lib = _lib.load()
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = getattr(lib, fn_name)(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                               _ptr(alpha), _ptr(S_in), _ptr(o), _ptr(S_out), _ptr(workspace),
                               ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, fn_name)


def _launch_stream(stream, device):
    return torch.cuda.current_stream(device) if stream is None else stream


def frame_scan_fwd(q, k, v, beta, alpha, S0=None, *, gates_are_logits: bool = False,
                   eps: float = 1e-6, normalize_keys: bool = True, reverse: bool = False,
                   o=None, S_final=None, workspace=None,
                   return_state: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Whole-clip frame-wise GDN scan.

    q, k: [B,F,N,H,D]; v: [B,F,N,H,D] (bf16 or fp32, all the same dtype);
    beta: [B,F,N,H] fp32; alpha: [B,F,H] fp32; S0: [B,H,D,D] fp32 or None.
    reverse=True runs the recurrence from the last frame to the first.
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
    desc = make_desc(B, H, F, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys, reverse=reverse)
    if o is not None:
        _check(o, "o", q.dtype, (B, F, N, H, D))
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, (B, H, D, D))
    _check_workspace(workspace, q.device)
    stream = _launch_stream(stream, q.device)
    # Buffers allocated here belong to the launch stream, so torch's caching
    # allocator never hands them to other work while the kernels still run.
    with torch.cuda.stream(stream):
        if o is None:
            o = torch.empty_like(q)
        if S_final is None and return_state:
            S_final = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(desc, q.device)
        _run("gdn_frame_scan_fwd", q, k, v, beta, alpha, S0, o, S_final, workspace, desc, stream)
    return o, S_final


def frame_scan_fwd_static(q, k, v, beta, alpha, S0=None, *, gates_are_logits: bool = False,
                          eps: float = 1e-6, normalize_keys: bool = True, reverse: bool = False,
                          o=None, S_final=None,
                          return_state: bool = True, stream=None):
    """frame_scan_fwd through gdn_frame_scan_fwd_static: the library's own static
    scratch instead of a workspace.  The C entry point allocates nothing; pass
    o and S_final to keep this wrapper from allocating them with torch."""
    B, F, N, H, D = q.shape
    _check(q, "q", q.dtype, (B, F, N, H, D))
    _check(k, "k", q.dtype, (B, F, N, H, D))
    _check(v, "v", q.dtype, (B, F, N, H, D))
    _check(beta, "beta", torch.float32, (B, F, N, H))
    _check(alpha, "alpha", torch.float32, (B, F, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, (B, H, D, D))
    if o is not None:
        _check(o, "o", q.dtype, (B, F, N, H, D))
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, (B, H, D, D))
    desc = make_desc(B, H, F, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys, reverse=reverse)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        if o is None:
            o = torch.empty_like(q)
        if S_final is None and return_state:
            S_final = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        st = _lib.load().gdn_frame_scan_fwd_static(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0),
            _ptr(o), _ptr(S_final), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_frame_scan_fwd_static")
    return o, S_final


def frame_scan_fwd_fp8(q, q_scale, k, k_scale, v, v_scale, beta, alpha, S0=None, *,
                       gates_are_logits: bool = False, eps: float = 1e-6, normalize_keys: bool = True,
                       reverse: bool = False, o=None, S_final=None, workspace=None,
                       return_state: bool = True, stream=None):
    """frame_scan_fwd on block-scaled FP8 inputs (OCP MXFP8, E4M3 elements).

    q, k, v: [B,F,N,H,D] torch.float8_e4m3fn; q_scale, k_scale, v_scale:
    [B,F,N,H,D/32] torch.uint8 E8M0 exponents (value = e4m3 * 2^(s - 127));
    D in {32, 64, 128}.  Returns (o [B,F,N,H,D] bfloat16, S_final fp32 or None).
    """
    B, F, N, H, D = q.shape
    f8 = torch.float8_e4m3fn
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, f8, (B, F, N, H, D))
    nb = D // 32
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check(t, name, torch.uint8, (B, F, N, H, nb))
    _check(beta, "beta", torch.float32, (B, F, N, H))
    _check(alpha, "alpha", torch.float32, (B, F, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, (B, H, D, D))
    if o is not None:
        _check(o, "o", torch.bfloat16, (B, F, N, H, D))
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, (B, H, D, D))
    _check_workspace(workspace, q.device)
    desc = make_desc(B, H, F, N, D, f8, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys, reverse=reverse)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):   # allocations belong to the launch stream
        if o is None:
            o = torch.empty((B, F, N, H, D), dtype=torch.bfloat16, device=q.device)
        if S_final is None and return_state:
            S_final = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(desc, q.device)
        ws_bytes = 0 if workspace is None else workspace.numel()
        st = _lib.load().gdn_frame_scan_fwd_fp8(
            ctypes.byref(desc), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale),
            _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S_final), _ptr(workspace),
            ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_frame_scan_fwd_fp8")
    return o, S_final


def frame_scan_fwd_fp4(q, q_scale, k, k_scale, v, v_scale, beta, alpha, S0=None, *,
                       gates_are_logits: bool = False, eps: float = 1e-6, normalize_keys: bool = True,
                       reverse: bool = False, o=None, S_final=None, workspace=None,
                       return_state: bool = True, stream=None):
    """frame_scan_fwd on block-scaled FP4 inputs (OCP MXFP4, E2M1 elements).

    q, k, v: [B,F,N,H,D/2] torch.uint8, two E2M1 codes per byte (feature 2j
    in the lower four bits of byte j); q_scale, k_scale, v_scale:
    [B,F,N,H,D/32] torch.uint8 E8M0 exponents; D in {32, 64, 128}.  Returns
    (o [B,F,N,H,D] bfloat16, S_final fp32 or None).
    """
    B, F, N, H, D2 = q.shape
    D = 2 * D2
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, torch.uint8, (B, F, N, H, D2))
    nb = D // 32
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check(t, name, torch.uint8, (B, F, N, H, nb))
    _check(beta, "beta", torch.float32, (B, F, N, H))
    _check(alpha, "alpha", torch.float32, (B, F, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, (B, H, D, D))
    if o is not None:
        _check(o, "o", torch.bfloat16, (B, F, N, H, D))
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, (B, H, D, D))
    _check_workspace(workspace, q.device)
    desc = make_desc(B, H, F, N, D, torch.bfloat16, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys, reverse=reverse)
    desc.io_dtype = _lib.GDN_FP4_E2M1
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):   # allocations belong to the launch stream
        if o is None:
            o = torch.empty((B, F, N, H, D), dtype=torch.bfloat16, device=q.device)
        if S_final is None and return_state:
            S_final = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(desc, q.device)
        ws_bytes = 0 if workspace is None else workspace.numel()
        st = _lib.load().gdn_frame_scan_fwd_fp4(
            ctypes.byref(desc), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale),
            _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S_final), _ptr(workspace),
            ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_frame_scan_fwd_fp4")
    return o, S_final


def frame_step(q, k, v, beta, alpha, S_in=None, *, gates_are_logits: bool = False,
               eps: float = 1e-6, normalize_keys: bool = True, o=None, S_out=None, workspace=None, stream=None):
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
    if o is not None:
        _check(o, "o", q.dtype, (B, 1, N, H, D))
    if S_out is not None:
        _check(S_out, "S_out", torch.float32, (B, H, D, D))
    _check_workspace(workspace, q.device)
    desc = make_desc(B, H, 1, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):   # allocations belong to the launch stream
        if o is None:
            o = torch.empty_like(q)
        if S_out is None:
            S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = alloc_workspace(desc, q.device)
        _run("gdn_frame_step", q, k, v, beta, alpha, S_in, o, S_out, workspace, desc, stream)
    return (o.squeeze(1) if squeeze else o), S_out


def workspace_size_bwd(desc: GdnDesc) -> int:
    return int(_lib.load().gdn_workspace_size_bwd(ctypes.byref(desc)))


def saved_size(desc: GdnDesc) -> int:
    return int(_lib.load().gdn_saved_size(ctypes.byref(desc)))


def workspace_size_bwd_saved(desc: GdnDesc) -> int:
    return int(_lib.load().gdn_workspace_size_bwd_saved(ctypes.byref(desc)))


def frame_scan_fwd_save(q, k, v, beta, alpha, S0=None, *, gates_are_logits: bool = False,
                        eps: float = 1e-6, normalize_keys: bool = True, reverse: bool = False,
                        o=None, S_final=None, saved=None, return_state: bool = True, stream=None):
    """frame_scan_fwd that also keeps, in `saved` (a uint8 device tensor of
    gdn_saved_size bytes, allocated when None), what frame_scan_bwd(...,
    saved=saved) reads instead of recomputing.  Returns (o, S_final, saved)."""
    B, F, N, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, (B, F, N, H, D))
    _check(beta, "beta", torch.float32, (B, F, N, H))
    _check(alpha, "alpha", torch.float32, (B, F, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, (B, H, D, D))
    if o is not None:
        _check(o, "o", q.dtype, (B, F, N, H, D))
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, (B, H, D, D))
    _check_workspace(saved, q.device)
    desc = make_desc(B, H, F, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys, reverse=reverse)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):   # allocations belong to the launch stream
        if o is None:
            o = torch.empty_like(q)
        if S_final is None and return_state:
            S_final = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        if saved is None:
            saved = torch.empty(max(saved_size(desc), 1), dtype=torch.uint8, device=q.device)
        st = _lib.load().gdn_frame_scan_fwd_save(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o),
            _ptr(S_final), _ptr(saved), ctypes.c_size_t(saved.numel()), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_frame_scan_fwd_save")
    return o, S_final, saved


def frame_scan_bwd(q, k, v, beta, alpha, dO, S0=None, dS_final=None, *, gates_are_logits: bool = False,
                   eps: float = 1e-6, normalize_keys: bool = True, reverse: bool = False,
                   workspace=None, return_dS0: bool = True, saved=None, stream=None):
    """Gradients of frame_scan_fwd with respect to its inputs.

    q, k, v, beta, alpha, S0 and the flags as for frame_scan_fwd; dO: [B,F,N,H,D]
    in the q dtype (the loss gradient of o); dS_final: [B,H,D,D] fp32 or None
    (zeros).  Returns (dq, dk, dv, dbeta, dalpha, dS0): dq, dk, dv in the q
    dtype, the rest fp32 (dbeta and dalpha are logit gradients with
    gates_are_logits; dS0 is None when return_dS0 is False).  With `saved`
    (from frame_scan_fwd_save on the same inputs) the per-frame operands of
    the forward walk are read from it instead of recomputed, and S0 is unused.
    """
    B, F, N, H, D = q.shape
    _check(q, "q", q.dtype, (B, F, N, H, D))
    _check(k, "k", q.dtype, (B, F, N, H, D))
    _check(v, "v", q.dtype, (B, F, N, H, D))
    _check(beta, "beta", torch.float32, (B, F, N, H))
    _check(alpha, "alpha", torch.float32, (B, F, H))
    _check(dO, "dO", q.dtype, (B, F, N, H, D))
    if S0 is not None:
        _check(S0, "S0", torch.float32, (B, H, D, D))
    if dS_final is not None:
        _check(dS_final, "dS_final", torch.float32, (B, H, D, D))
    _check_workspace(workspace, q.device)
    desc = make_desc(B, H, F, N, D, q.dtype, gates_are_logits=gates_are_logits, eps=eps,
                     normalize_keys=normalize_keys, reverse=reverse)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):   # allocations belong to the launch stream
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dbeta, dalpha = torch.empty_like(beta), torch.empty_like(alpha)
        dS0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device) if return_dS0 else None
        lib = _lib.load()
        if workspace is None:
            n = workspace_size_bwd_saved(desc) if saved is not None else workspace_size_bwd(desc)
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
        ws_bytes = 0 if workspace is None else workspace.numel()
        if saved is not None:
            name = "gdn_frame_scan_bwd_saved"
            st = lib.gdn_frame_scan_bwd_saved(
                ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(dO),
                _ptr(dS_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dalpha), _ptr(dS0),
                _ptr(saved), ctypes.c_size_t(saved.numel()), _ptr(workspace), ctypes.c_size_t(ws_bytes),
                ctypes.c_void_p(stream.cuda_stream))
        else:
            name = "gdn_frame_scan_bwd"
            st = lib.gdn_frame_scan_bwd(
                ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(dO),
                _ptr(dS_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dalpha), _ptr(dS0),
                _ptr(workspace), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, name)
    return dq, dk, dv, dbeta, dalpha, dS0


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


def block_workspace_size(B, H, F, N, D, C) -> int:
    desc = make_desc(B, H, F, N, D, torch.bfloat16)
    return int(_lib.load().gdn_block_workspace_size(ctypes.byref(desc), int(C)))


def block_in_proj(x, w_qkv, w_gate, *, H: int, D: int, q=None, k=None, v=None, beta_logit=None,
                  alpha_logit=None, workspace=None, stream=None):
    """Input projections of a GDN block: hidden states to the scan's inputs.

    x: [B,F,N,C] bf16; w_qkv: [3,H,D,C] bf16; w_gate: [2,H,C] bf16 (weights
    output-major, as torch.nn.Linear stores them).  Returns
    (q, k, v, beta_logit, alpha_logit): q, k, v [B,F,N,H,D] bf16,
    beta_logit [B,F,N,H] fp32 (one per token) and alpha_logit [B,F,H] fp32
    (the frame mean of the per-token alpha terms); the logits feed
    frame_scan_fwd(..., gates_are_logits=True).
    """
    B, F, N, C = x.shape
    _check(x, "x", torch.bfloat16, (B, F, N, C))
    _check(w_qkv, "w_qkv", torch.bfloat16, (3, H, D, C))
    _check(w_gate, "w_gate", torch.bfloat16, (2, H, C))
    outs = {"q": q, "k": k, "v": v}
    for name, t in outs.items():
        if t is not None:
            _check(t, name, torch.bfloat16, (B, F, N, H, D))
    if beta_logit is not None:
        _check(beta_logit, "beta_logit", torch.float32, (B, F, N, H))
    if alpha_logit is not None:
        _check(alpha_logit, "alpha_logit", torch.float32, (B, F, H))
    _check_workspace(workspace, x.device)
    desc = make_desc(B, H, F, N, D, torch.bfloat16)
    lib = _lib.load()
    stream = _launch_stream(stream, x.device)
    with torch.cuda.stream(stream):   # allocations belong to the launch stream
        q, k, v = [t if t is not None else torch.empty((B, F, N, H, D), dtype=torch.bfloat16, device=x.device)
                   for t in (q, k, v)]
        if beta_logit is None:
            beta_logit = torch.empty((B, F, N, H), dtype=torch.float32, device=x.device)
        if alpha_logit is None:
            alpha_logit = torch.empty((B, F, H), dtype=torch.float32, device=x.device)
        if workspace is None:
            n = int(lib.gdn_block_workspace_size(ctypes.byref(desc), int(C)))
            workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
        st = lib.gdn_block_in_proj(ctypes.byref(desc), int(C), _ptr(x), _ptr(w_qkv), _ptr(w_gate), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(beta_logit), _ptr(alpha_logit), _ptr(workspace),
                                   ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_block_in_proj")
    return q, k, v, beta_logit, alpha_logit


def block_out_proj(o, w_out, *, y=None, workspace=None, stream=None):
    """Output projection of a GDN block: y [B,F,N,C] bf16 = o [B,F,N,H,D] bf16
    (flattened to H*D) times the transpose of w_out [C, H*D] bf16."""
    B, F, N, H, D = o.shape
    C = w_out.shape[0]
    _check(o, "o", torch.bfloat16, (B, F, N, H, D))
    _check(w_out, "w_out", torch.bfloat16, (C, H * D))
    if y is not None:
        _check(y, "y", torch.bfloat16, (B, F, N, C))
    _check_workspace(workspace, o.device)
    desc = make_desc(B, H, F, N, D, torch.bfloat16)
    lib = _lib.load()
    stream = _launch_stream(stream, o.device)
    with torch.cuda.stream(stream):
        if y is None:
            y = torch.empty((B, F, N, C), dtype=torch.bfloat16, device=o.device)
        if workspace is None:
            n = int(lib.gdn_block_workspace_size(ctypes.byref(desc), int(C)))
            workspace = torch.empty(n, dtype=torch.uint8, device=o.device)
        st = lib.gdn_block_out_proj(ctypes.byref(desc), int(C), _ptr(o), _ptr(w_out), _ptr(y), _ptr(workspace),
                                    ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise GdnError(st, "gdn_block_out_proj")
    return y
