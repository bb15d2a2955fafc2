"""ctypes loader for libgdn.so (the C ABI declared in include/gdn.h).

There is no fallback: if the HIP library is missing or fails to load, every
entry point raises.  Build it with ``python -m gated_deltanet_scan_amd.build``
(or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_BF16 = 0
GDN_F32 = 1
GDN_FP8_E4M3 = 2
GDN_FP4_E2M1 = 3
GDN_FLAG_GATES_ARE_LOGITS = 0x1
GDN_FLAG_NO_KEY_NORM = 0x2
GDN_FLAG_REVERSE = 0x4
GDN_NUM_KERNELS = 9

STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_ALIGNMENT",
          4: "GDN_ERR_ALIAS", 5: "GDN_ERR_WORKSPACE", 6: "GDN_ERR_LAUNCH", 7: "GDN_ERR_NO_DEVICE"}


class GdnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("F", ctypes.c_int32),
                ("N", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("eps", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib_or_none_status_string(status)
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), msg))


_lib = None


def _lib_or_none_status_string(status):
    try:
        return load().gdn_status_string(status).decode()
    except Exception:  # pragma: no cover
        return "?"


def load():
    """Load libgdn.so once; raise OSError with a build hint when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError("libgdn.so not built at %s; run `python -m gated_deltanet_scan_amd.build`"
                      % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(GdnDesc)
    fp = ctypes.c_void_p
    lib.gdn_workspace_size.argtypes = [dp]
    lib.gdn_workspace_size.restype = sz
    for name in ("gdn_frame_scan_fwd", "gdn_frame_step"):
        fn = getattr(lib, name)
        fn.argtypes = [dp, vp, vp, vp, fp, fp, fp, vp, fp, vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.gdn_workspace_size_bwd.argtypes = [dp]
    lib.gdn_workspace_size_bwd.restype = sz
    lib.gdn_frame_scan_bwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp, vp, sz, vp]
    lib.gdn_frame_scan_bwd.restype = ctypes.c_int
    lib.gdn_saved_size.argtypes = [dp]
    lib.gdn_saved_size.restype = sz
    lib.gdn_workspace_size_bwd_saved.argtypes = [dp]
    lib.gdn_workspace_size_bwd_saved.restype = sz
    lib.gdn_frame_scan_fwd_save.argtypes = [dp, vp, vp, vp, fp, fp, fp, vp, fp, vp, sz, vp]
    lib.gdn_frame_scan_fwd_save.restype = ctypes.c_int
    lib.gdn_frame_scan_bwd_saved.argtypes = [dp, vp, vp, vp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp, vp, sz, vp, sz,
                                             vp]
    lib.gdn_frame_scan_bwd_saved.restype = ctypes.c_int
    lib.gdn_frame_scan_fwd_fp8.argtypes = [dp, vp, vp, vp, vp, vp, vp, fp, fp, fp, vp, fp, vp, sz, vp]
    lib.gdn_frame_scan_fwd_fp8.restype = ctypes.c_int
    lib.gdn_frame_scan_fwd_fp4.argtypes = [dp, vp, vp, vp, vp, vp, vp, fp, fp, fp, vp, fp, vp, sz, vp]
    lib.gdn_frame_scan_fwd_fp4.restype = ctypes.c_int
    lib.gdn_block_workspace_size.argtypes = [dp, ctypes.c_int32]
    lib.gdn_block_workspace_size.restype = sz
    lib.gdn_block_in_proj.argtypes = [dp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, fp, fp, vp, sz, vp]
    lib.gdn_block_in_proj.restype = ctypes.c_int
    lib.gdn_block_out_proj.argtypes = [dp, ctypes.c_int32, vp, vp, vp, vp, sz, vp]
    lib.gdn_block_out_proj.restype = ctypes.c_int
    lib.gdn_frame_scan_fwd_static.argtypes = [dp, vp, vp, vp, fp, fp, fp, vp, fp, vp]
    lib.gdn_frame_scan_fwd_static.restype = ctypes.c_int
    lib.gdn_static_scratch_bytes.argtypes = []
    lib.gdn_static_scratch_bytes.restype = sz
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_int32
    lib.gdn_profile_begin.argtypes = []
    lib.gdn_profile_begin.restype = ctypes.c_int
    lib.gdn_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.gdn_profile_end.restype = ctypes.c_int
    lib.gdn_kernel_name.argtypes = [ctypes.c_int32]
    lib.gdn_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib
