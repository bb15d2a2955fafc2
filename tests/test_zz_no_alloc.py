"""The allocation-free entry point against the workspace entry point.

gdn_frame_scan_fwd_static runs the scan with the library's static scratch
(64 MiB per GPU) in place of a caller workspace, chunking the frames to fit
it.  Called here through the C ABI on two calls in a row, the second with a
smaller input: its outputs must equal gdn_frame_scan_fwd's (the state crosses
chunk boundaries in fp32, so the bits agree), which also meets the oracle
tolerance that gdn_frame_scan_fwd is held to.
"""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_scan_amd import _lib, api, inputs
from test_gpu_parity import check

pytestmark = pytest.mark.gpu


def call_static(w):
    lib = _lib.load()
    q, k, v, b, a, s0 = inputs.to_torch(w, "cuda")
    o = torch.full_like(q, float("nan"))
    S = torch.full((w.B, w.H, w.Dv, w.Dk), float("nan"), dtype=torch.float32, device="cuda")
    desc = api.make_desc(w.B, w.H, w.F, w.N, w.Dk, q.dtype)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.gdn_frame_scan_fwd_static(ctypes.byref(desc), ptr(q), ptr(k), ptr(v), ptr(b), ptr(a),
                                       ptr(s0), ptr(o), ptr(S),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.STATUS.get(st, st)
    o2, S2 = api.frame_scan_fwd(q, k, v, b, a, s0)
    torch.cuda.synchronize()
    return o, S, o2, S2


def test_static_scratch_matches_workspace_entry_point():
    # 1) the full-minute shape: 16 (b, h) x 160 KiB per frame, so the 64 MiB
    #    scratch takes 25 frames per chunk and the scan runs in five chunks
    w1 = inputs.make(1, 16, 121, 880, 128, dtype="bf16", seed=61, s0_std=0.02)
    # 2) then a smaller input on the same scratch (one chunk, d = 64)
    w2 = inputs.make(2, 4, 6, 200, 64, dtype="bf16", seed=62, s0_std=0.05)
    for w in (w1, w2):
        o, S, o2, S2 = call_static(w)
        check(o.float().cpu().numpy(), o2.float().cpu().numpy(), "bf16", "O static vs workspace")
        check(S.cpu().numpy(), S2.cpu().numpy(), "bf16", "S static vs workspace")
        assert torch.equal(o, o2) and torch.equal(S, S2)
