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
    assert [lib.gdn_kernel_name(i) for i in range(5)] == [b"frame_gram", b"state_scan",
                                                          b"frame_output", b"state_copy",
                                                          b"frame_step"]
    assert lib.gdn_kernel_name(5) is None and lib.gdn_kernel_name(-1) is None


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
    ms = (ctypes.c_double * 5)()
    n = (ctypes.c_int64 * 5)()
    assert lib.gdn_profile_end(ms, n) == OK
    assert list(n) == [0] * 5 and list(ms) == [0.0] * 5
