"""The C ABI on the host: the library loads, exports everything include/gdn.h
declares, and rejects bad calls with the documented status before launching.

Every call here fails a host-side check (or has nothing to compute), so no
pointer is ever dereferenced and no kernel is launched; the fake addresses are
never touched.
"""
import ctypes
import os
import re

import pytest

from gated_deltanet_scan_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, ALIGN, ALIAS, WORKSPACE = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from gated_deltanet_scan_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdn_frame_scan_fwd", "gdn_frame_step", "gdn_workspace_size",
            "gdn_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "libgdn.so does not export %s" % n


def test_status_strings_and_version(lib):
    for s in range(8):
        assert lib.gdn_status_string(s)
    assert lib.gdn_status_string(99) == b"unknown status"
    assert lib.gdn_version() >= 10000
    assert [lib.gdn_kernel_name(i) for i in range(9)] == [b"frame_gram", b"state_scan",
                                                          b"frame_output", b"state_copy",
                                                          b"frame_step", b"w_gram", b"adjoint_scan",
                                                          b"frame_dq", b"frame_dkv"]
    assert lib.gdn_kernel_name(9) is None and lib.gdn_kernel_name(-1) is None


def desc(B=1, H=2, F=3, N=5, D=16, io=_lib.GDN_BF16, flags=0, eps=1e-6, Dv=None):
    return _lib.GdnDesc(B, H, F, N, D, D if Dv is None else Dv, io, flags, eps)


def test_workspace_size(lib):
    # per (b, h, frame): Gm, U and the state S_f for frame_output (bf16:
    # 2 + 4 + 4 bytes per matrix entry, S_f as bf16 plus a one-byte remainder
    # code in room for two; fp32: 4 + 4 + 4), rounded to 256 bytes, then one
    # fp32 carry state per (b, h)
    for io, per_entry in ((_lib.GDN_BF16, 10), (_lib.GDN_F32, 12)):
        d = desc(B=2, H=3, F=5, N=7, D=64, io=io)
        per_frames = 2 * 3 * 5 * per_entry * 64 * 64
        assert lib.gdn_workspace_size(ctypes.byref(d)) == \
            (per_frames + 255) // 256 * 256 + 2 * 3 * 64 * 64 * 4
    # one frame: fp32 partial G and U (8*D*D bytes) per (b, h, token range),
    # ranges of whole 64-token stages sized for 256 CUs (here 128 units: two
    # ranges each), rounded to 256 bytes, then a copy of S_in
    d = desc(B=4, H=32, F=1, N=880, D=64)
    assert lib.gdn_workspace_size(ctypes.byref(d)) == 4 * 32 * 2 * 8 * 64 * 64 + 4 * 32 * 64 * 64 * 4
    d = desc(B=1, H=1, F=1, N=880, D=128)          # one unit: ceil(880/64) = 14 ranges
    assert lib.gdn_workspace_size(ctypes.byref(d)) == 14 * 8 * 128 * 128 + 128 * 128 * 4
    assert lib.gdn_workspace_size(ctypes.byref(desc(D=48))) == 0
    assert lib.gdn_workspace_size(None) == 0
    assert lib.gdn_workspace_size(ctypes.byref(desc(F=0))) == 0


# fake, never-dereferenced device addresses, 256-byte aligned and far apart
BASE = 0x7f0000000000
P = {n: BASE + i * (1 << 32) for i, n in enumerate(["q", "k", "v", "beta", "alpha", "S0", "o",
                                                      "S_final", "ws"])}


def call(lib, d, fn="gdn_frame_scan_fwd", ws_bytes=1 << 40, **over):
    p = dict(P)
    p.update(over)
    args = [p[n] for n in ["q", "k", "v", "beta", "alpha", "S0", "o", "S_final", "ws"]]
    return getattr(lib, fn)(None if d is None else ctypes.byref(d), *args,
                            ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("d,expect", [
    (None, INVALID),
    (desc(B=-1), INVALID),
    (desc(N=-2), INVALID),
    (desc(io=7), INVALID),
    (desc(flags=0x80), INVALID),
    (desc(eps=0.0), INVALID),
    (desc(eps=float("nan")), INVALID),
    (desc(D=48), UNSUPPORTED),
    (desc(D=256), UNSUPPORTED),
    (desc(D=64, Dv=128), UNSUPPORTED),
])
def test_descriptor_errors(lib, d, expect):
    assert call(lib, d) == expect


def test_missing_pointers(lib):
    d = desc()
    for n in ["q", "k", "v", "beta", "alpha", "o"]:
        assert call(lib, d, **{n: None}) == INVALID, n


def test_alignment(lib):
    d = desc()
    for n in ["q", "k", "v", "o", "S0", "S_final"]:
        assert call(lib, d, **{n: P[n] + 8}) == ALIGN, n
    for n in ["beta", "alpha"]:
        assert call(lib, d, **{n: P[n] + 2}) == ALIGN, n
    assert call(lib, d, ws=P["ws"] + 16) == ALIGN


def test_workspace_errors(lib):
    d = desc()
    need = lib.gdn_workspace_size(ctypes.byref(d))
    assert call(lib, d, ws_bytes=need - 1) == WORKSPACE
    assert call(lib, d, ws=None) == WORKSPACE


def test_aliasing(lib):
    d = desc()
    assert call(lib, d, o=P["q"]) == ALIAS
    assert call(lib, d, o=P["v"] + 64) == ALIAS                   # partial overlap
    assert call(lib, d, S_final=P["o"]) == ALIAS
    assert call(lib, d, S_final=P["alpha"]) == ALIAS
    assert call(lib, d, S_final=P["S0"] + 16) == ALIAS             # only exact in-place is allowed
    assert call(lib, d, ws=P["k"]) == ALIAS
    assert call(lib, d, ws=P["o"]) == ALIAS


def test_step_errors(lib):
    assert call(lib, desc(F=2), fn="gdn_frame_step") == INVALID
    assert call(lib, desc(F=1), fn="gdn_frame_step", S_final=None) == INVALID


def test_empty_calls_do_nothing(lib):
    # nothing to compute: accepted without touching any pointer or device
    assert call(lib, desc(B=0), q=None, k=None, v=None, beta=None, alpha=None, o=None) == OK
    assert call(lib, desc(H=0), q=None, k=None, v=None, beta=None, alpha=None, o=None) == OK
    assert call(lib, desc(F=0), S_final=None, q=None, k=None, v=None, beta=None, alpha=None,
                o=None, ws=None) == OK


def test_profile_session_without_launches(lib):
    assert lib.gdn_profile_begin() == OK
    ms = (ctypes.c_double * _lib.GDN_NUM_KERNELS)()
    n = (ctypes.c_int64 * _lib.GDN_NUM_KERNELS)()
    assert lib.gdn_profile_end(ms, n) == OK
    assert list(n) == [0] * _lib.GDN_NUM_KERNELS and list(ms) == [0.0] * _lib.GDN_NUM_KERNELS


def test_static_scratch_rejects_what_does_not_fit(lib):
    """gdn_frame_scan_fwd_static: the scratch holds at least one frame for
    moderate shapes; a shape whose single frame of operands exceeds it is
    refused on the host before any launch (no pointer is touched)."""
    assert lib.gdn_static_scratch_bytes() == 64 << 20
    # B1 H512 d128: one frame of workspace items is 512 x 160 KiB = 80 MiB
    d = desc(B=1, H=512, F=2, N=1, D=128)
    p = [P[n] for n in ["q", "k", "v", "beta", "alpha", "S0", "o", "S_final"]]
    assert lib.gdn_frame_scan_fwd_static(ctypes.byref(d), *p, None) == WORKSPACE
    # invalid descriptors report as for the workspace entry point
    assert lib.gdn_frame_scan_fwd_static(None, *p, None) == INVALID
    assert lib.gdn_frame_scan_fwd_static(ctypes.byref(desc(D=48)), *p, None) == UNSUPPORTED
    # nothing to compute: accepted without touching any pointer
    d0 = desc(B=0)
    assert lib.gdn_frame_scan_fwd_static(ctypes.byref(d0), None, None, None, None, None, None,
                                         None, None, None) == OK


# ---------------------------------------------------------------- backward entry point
BWD_NAMES = ["q", "k", "v", "beta", "alpha", "S0", "dO", "dS_final", "dq", "dk", "dv", "dbeta", "dalpha",
             "dS0", "ws"]
PB = {n: BASE + i * (1 << 32) for i, n in enumerate(BWD_NAMES)}


def call_bwd(lib, d, ws_bytes=1 << 40, **over):
    p = dict(PB)
    p.update(over)
    return lib.gdn_frame_scan_bwd(None if d is None else ctypes.byref(d), *[p[n] for n in BWD_NAMES],
                                  ctypes.c_size_t(ws_bytes), None)


def test_bwd_workspace_size(lib):
    # two item sets (forward: Gm, U, S planes; backward: W and the X planes),
    # each rounded to 256 bytes, the states entering launch chunks 1.. and one
    # carried gradient state, all per (b, h), then a key scale per token
    # (rounded to 256 bytes)
    r256 = lambda x: (x + 255) // 256 * 256
    for io, per_entry in ((_lib.GDN_BF16, 10), (_lib.GDN_F32, 12)):
        d = desc(B=2, H=3, F=5, N=7, D=64, io=io)
        per_set = r256(2 * 3 * 5 * per_entry * 64 * 64)
        assert lib.gdn_workspace_size_bwd(ctypes.byref(d)) == \
            2 * per_set + 2 * 3 * 64 * 64 * 4 + r256(2 * 5 * 7 * 3 * 4)
    # D = 16: each plane's fragments are padded to a 32-wide contraction, so an
    # item is 4 KiB (1 KiB each for Gm, the S plane and its codes, U); chunks
    # of 256 and 44 frames
    d = desc(B=1, H=2, F=300, N=5, D=16)
    per_set = r256(2 * 256 * 4096)
    assert lib.gdn_workspace_size_bwd(ctypes.byref(d)) == 2 * per_set + 2 * (2 * 16 * 16 * 4) + r256(300 * 5 * 2 * 4)
    assert lib.gdn_workspace_size_bwd(ctypes.byref(desc(D=48))) == 0
    assert lib.gdn_workspace_size_bwd(None) == 0


@pytest.mark.parametrize("d,expect", [
    (None, INVALID), (desc(B=-1), INVALID), (desc(flags=0x80), INVALID), (desc(D=48), UNSUPPORTED),
])
def test_bwd_descriptor_errors(lib, d, expect):
    assert call_bwd(lib, d) == expect


def test_bwd_pointer_alignment_workspace(lib):
    d = desc()
    for n in ["q", "k", "v", "beta", "alpha", "dO", "dq", "dk", "dv", "dbeta", "dalpha"]:
        assert call_bwd(lib, d, **{n: None}) == INVALID, n
    for n in ["q", "k", "v", "dO", "dq", "dk", "dv", "S0", "dS_final", "dS0"]:
        assert call_bwd(lib, d, **{n: PB[n] + 8}) == ALIGN, n
    for n in ["beta", "alpha", "dbeta", "dalpha"]:
        assert call_bwd(lib, d, **{n: PB[n] + 2}) == ALIGN, n
    need = lib.gdn_workspace_size_bwd(ctypes.byref(d))
    assert call_bwd(lib, d, ws_bytes=need - 1) == WORKSPACE
    assert call_bwd(lib, d, ws=None) == WORKSPACE


def test_bwd_aliasing(lib):
    d = desc()
    assert call_bwd(lib, d, dq=PB["q"]) == ALIAS
    assert call_bwd(lib, d, dk=PB["dO"] + 64) == ALIAS
    assert call_bwd(lib, d, dv=PB["dk"]) == ALIAS
    assert call_bwd(lib, d, dalpha=PB["alpha"]) == ALIAS
    assert call_bwd(lib, d, dbeta=PB["ws"]) == ALIAS
    assert call_bwd(lib, d, dS0=PB["S0"]) == ALIAS
    assert call_bwd(lib, d, dS0=PB["dS_final"] + 16) == ALIAS        # only exact in-place is allowed
    assert call_bwd(lib, desc(B=0), **{n: None for n in BWD_NAMES}) == OK


# ---------------------------------------------------------------- block-scaled FP8 entry point
FP8_NAMES = ["q", "qs", "k", "ks", "v", "vs", "beta", "alpha", "S0", "o", "S_final", "ws"]
P8 = {n: BASE + i * (1 << 32) for i, n in enumerate(FP8_NAMES)}


def call_fp8(lib, d, ws_bytes=1 << 40, **over):
    p = dict(P8)
    p.update(over)
    return lib.gdn_frame_scan_fwd_fp8(None if d is None else ctypes.byref(d), *[p[n] for n in FP8_NAMES[:-1]],
                                      p["ws"], ctypes.c_size_t(ws_bytes), None)


def test_fp8_entry_point_checks(lib):
    f8 = _lib.GDN_FP8_E4M3
    assert call_fp8(lib, desc(D=16, io=f8)) == UNSUPPORTED           # one 32-feature scale block at least
    assert call_fp8(lib, desc(D=64, io=_lib.GDN_BF16)) == INVALID      # this entry point takes FP8 only
    for n in ["q", "qs", "k", "ks", "v", "vs", "beta", "alpha", "o"]:
        assert call_fp8(lib, desc(D=64, io=f8), **{n: None}) == INVALID, n
    assert call_fp8(lib, desc(D=64, io=f8), o=P8["q"]) == ALIAS
    assert call_fp8(lib, desc(D=64, io=f8), o=P8["ks"]) == ALIAS
    assert call_fp8(lib, desc(D=64, io=f8), ws=P8["vs"]) == ALIAS
    need = lib.gdn_workspace_size(ctypes.byref(desc(D=64, io=f8)))
    assert need == lib.gdn_workspace_size(ctypes.byref(desc(D=64, io=_lib.GDN_BF16)))
    assert call_fp8(lib, desc(D=64, io=f8), ws_bytes=need - 1) == WORKSPACE
    # the other entry points refuse the FP8 dtype (they have no scales)
    assert call(lib, desc(D=64, io=f8)) == INVALID
    assert call_bwd(lib, desc(D=64, io=f8)) == UNSUPPORTED


def call_fp4(lib, d, ws_bytes=1 << 40, **over):
    p = dict(P8)
    p.update(over)
    return lib.gdn_frame_scan_fwd_fp4(None if d is None else ctypes.byref(d), *[p[n] for n in FP8_NAMES[:-1]],
                                      p["ws"], ctypes.c_size_t(ws_bytes), None)


def test_fp4_entry_point_checks(lib):
    f4 = _lib.GDN_FP4_E2M1
    assert call_fp4(lib, desc(D=16, io=f4)) == UNSUPPORTED
    assert call_fp4(lib, desc(D=64, io=_lib.GDN_FP8_E4M3)) == INVALID   # each MX entry point takes its own format
    assert call_fp8(lib, desc(D=64, io=f4)) == INVALID
    for n in ["q", "qs", "k", "ks", "v", "vs", "beta", "alpha", "o"]:
        assert call_fp4(lib, desc(D=64, io=f4), **{n: None}) == INVALID, n
    # q holds 2*3*5 tokens of 64 features at half a byte each: 960 bytes
    assert call_fp4(lib, desc(D=64, io=f4), o=P8["q"] + 944) == ALIAS      # 16-byte aligned, inside q
    assert call_fp4(lib, desc(D=64, io=f4), S_final=P8["vs"]) == ALIAS
    assert call_fp4(lib, desc(D=64, io=f4), ws=P8["ks"]) == ALIAS
    need = lib.gdn_workspace_size(ctypes.byref(desc(D=64, io=f4)))
    assert need == lib.gdn_workspace_size(ctypes.byref(desc(D=64, io=_lib.GDN_BF16)))
    assert call_fp4(lib, desc(D=64, io=f4), ws_bytes=need - 1) == WORKSPACE
    assert call(lib, desc(D=64, io=f4)) == INVALID
    assert call_bwd(lib, desc(D=64, io=f4)) == UNSUPPORTED


# ----------------------------------------------------------- block projections
BP = {n: BASE + i * (1 << 32) for i, n in enumerate(["x", "w_qkv", "w_gate", "q", "k", "v", "bl", "al", "ws",
                                                       "o", "w_out", "y"])}


def call_in(lib, d, C=64, ws_bytes=1 << 40, **over):
    p = dict(BP)
    p.update(over)
    return lib.gdn_block_in_proj(None if d is None else ctypes.byref(d), C,
                                 *[p[n] for n in ["x", "w_qkv", "w_gate", "q", "k", "v", "bl", "al", "ws"]],
                                 ctypes.c_size_t(ws_bytes), None)


def call_out(lib, d, C=64, ws_bytes=1 << 40, **over):
    p = dict(BP)
    p.update(over)
    return lib.gdn_block_out_proj(None if d is None else ctypes.byref(d), C, p["o"], p["w_out"], p["y"], p["ws"],
                                  ctypes.c_size_t(ws_bytes), None)


def test_block_workspace_size(lib):
    d = desc(B=2, H=3, F=5, N=7, D=16)
    # 32 MiB for the GEMM library plus fp32 partial sums of the alpha terms per
    # (b, f, 64-token chunk, h), rounded to 256 bytes
    assert lib.gdn_block_workspace_size(ctypes.byref(d), 64) == (32 << 20) + 256
    d = desc(B=1, H=16, F=121, N=880, D=128)
    assert lib.gdn_block_workspace_size(ctypes.byref(d), 2048) == (32 << 20) + (121 * 14 * 16 * 4 + 255) // 256 * 256
    assert lib.gdn_block_workspace_size(ctypes.byref(d), 12) == 0          # C not a multiple of 8
    assert lib.gdn_block_workspace_size(None, 64) == 0


@pytest.mark.parametrize("d,C,expect", [
    (None, 64, INVALID),
    (desc(B=-1), 64, INVALID),
    (desc(H=0), 64, INVALID),
    (desc(), 0, INVALID),
    (desc(io=_lib.GDN_F32), 64, UNSUPPORTED),
    (desc(D=64, Dv=32), 64, UNSUPPORTED),
    (desc(), 60, UNSUPPORTED),                  # C not a multiple of 8
    (desc(H=1, D=12), 64, UNSUPPORTED),         # H*D not a multiple of 8
    (desc(), (1 << 20) + 8, UNSUPPORTED),       # wider than 2^20
])
def test_block_descriptor_errors(lib, d, C, expect):
    assert call_in(lib, d, C) == expect
    assert call_out(lib, d, C) == expect


def test_block_pointer_checks(lib):
    d = desc()
    for n in ["x", "w_qkv", "w_gate", "q", "k", "v", "bl", "al"]:
        assert call_in(lib, d, **{n: None}) == INVALID, n
    for n in ["x", "w_qkv", "w_gate", "q", "k", "v"]:
        assert call_in(lib, d, **{n: BP[n] + 8}) == ALIGN, n
    assert call_in(lib, d, bl=BP["bl"] + 2) == ALIGN
    assert call_in(lib, d, ws=BP["ws"] + 16) == ALIGN
    assert call_in(lib, d, ws=None) == WORKSPACE
    need = lib.gdn_block_workspace_size(ctypes.byref(d), 64)
    assert call_in(lib, d, ws_bytes=need - 1) == WORKSPACE
    assert call_in(lib, d, q=BP["x"]) == ALIAS
    assert call_in(lib, d, k=BP["q"] + 16) == ALIAS
    assert call_in(lib, d, al=BP["ws"] + 1024) == ALIAS
    for n in ["o", "w_out", "y"]:
        assert call_out(lib, d, **{n: None}) == INVALID, n
        assert call_out(lib, d, **{n: BP[n] + 8}) == ALIGN, n
    assert call_out(lib, d, y=BP["o"]) == ALIAS
    assert call_out(lib, d, y=BP["ws"] + 4096) == ALIAS
    assert call_out(lib, d, ws_bytes=need - 1) == WORKSPACE


# ------------------------------------------------------------ saved states
def test_saved_sizes(lib):
    d = desc(B=2, H=3, F=5, N=7, D=64)
    item = 10 * 64 * 64                                   # bf16 item: Gm, U, S planes
    per_set = (2 * 3 * 5 * item + 255) // 256 * 256       # one chunk of items
    state = (2 * 3 * 64 * 64 * 4 + 255) // 256 * 256
    rho = (2 * 5 * 7 * 3 * 4 + 255) // 256 * 256
    assert lib.gdn_saved_size(ctypes.byref(d)) == per_set + state + rho
    assert lib.gdn_workspace_size_bwd_saved(ctypes.byref(d)) == per_set + state
    # two chunks of at most 256 frames: two item sets and two entering states
    d = desc(B=1, H=2, F=300, N=5, D=16)
    item16 = lib.gdn_saved_size(ctypes.byref(desc(B=1, H=1, F=1, N=0, D=16))) - 16 * 16 * 4
    assert item16 > 0
    s2 = lib.gdn_saved_size(ctypes.byref(d))
    assert s2 == 2 * ((2 * 256 * item16 + 255) // 256 * 256) + 2 * ((2 * 16 * 16 * 4 + 255) // 256 * 256) + \
        (300 * 5 * 2 * 4 + 255) // 256 * 256
    assert lib.gdn_saved_size(ctypes.byref(desc(F=0))) == 0
    assert lib.gdn_saved_size(ctypes.byref(desc(io=_lib.GDN_FP8_E4M3, D=32))) == 0
    assert lib.gdn_saved_size(None) == 0


SV = {n: BASE + i * (1 << 32) for i, n in enumerate(["q", "k", "v", "beta", "alpha", "S0", "o", "S_final", "saved",
                                                       "dO", "dS", "dq", "dk", "dv", "db", "da", "dS0", "ws"])}


def call_save(lib, d, sv_bytes=1 << 40, **over):
    p = dict(SV)
    p.update(over)
    return lib.gdn_frame_scan_fwd_save(None if d is None else ctypes.byref(d),
                                       *[p[n] for n in ["q", "k", "v", "beta", "alpha", "S0", "o", "S_final", "saved"]],
                                       ctypes.c_size_t(sv_bytes), None)


def call_bwd_saved(lib, d, sv_bytes=1 << 40, ws_bytes=1 << 40, **over):
    p = dict(SV)
    p.update(over)
    return lib.gdn_frame_scan_bwd_saved(None if d is None else ctypes.byref(d),
                                        *[p[n] for n in ["q", "k", "v", "beta", "alpha", "dO", "dS", "dq", "dk", "dv",
                                                         "db", "da", "dS0", "saved"]],
                                        ctypes.c_size_t(sv_bytes), p["ws"], ctypes.c_size_t(ws_bytes), None)


def test_saved_entry_checks(lib):
    d = desc()
    need = lib.gdn_saved_size(ctypes.byref(d))
    assert call_save(lib, None) == INVALID
    assert call_save(lib, desc(io=_lib.GDN_FP8_E4M3, D=32)) == UNSUPPORTED
    assert call_save(lib, d, saved=None) == WORKSPACE
    assert call_save(lib, d, sv_bytes=need - 1) == WORKSPACE
    assert call_save(lib, d, saved=SV["saved"] + 16) == ALIGN
    assert call_save(lib, d, q=None) == INVALID
    assert call_save(lib, d, o=SV["o"] + 8) == ALIGN
    assert call_save(lib, d, saved=SV["q"]) == ALIAS
    assert call_save(lib, d, o=SV["saved"] + 4096) == ALIAS
    assert call_save(lib, d, S_final=SV["saved"]) == ALIAS
    assert call_bwd_saved(lib, None) == INVALID
    assert call_bwd_saved(lib, desc(io=_lib.GDN_FP8_E4M3, D=32)) == UNSUPPORTED
    assert call_bwd_saved(lib, d, saved=None) == WORKSPACE
    assert call_bwd_saved(lib, d, sv_bytes=need - 1) == WORKSPACE
    wneed = lib.gdn_workspace_size_bwd_saved(ctypes.byref(d))
    assert call_bwd_saved(lib, d, ws_bytes=wneed - 1) == WORKSPACE
    assert call_bwd_saved(lib, d, ws=None) == WORKSPACE
    assert call_bwd_saved(lib, d, saved=SV["saved"] + 16) == ALIGN
    assert call_bwd_saved(lib, d, dq=SV["saved"]) == ALIAS          # saved is an input
    assert call_bwd_saved(lib, d, ws=SV["saved"] + 256) == ALIAS
    assert call_bwd_saved(lib, d, dk=SV["q"]) == ALIAS
