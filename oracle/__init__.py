"""fp64 CPU oracle of the frame-wise Gated DeltaNet forward scan.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The HIP library never imports or
links anything here, and nothing here imports the HIP library.

The arithmetic lives in ``gdn_oracle.c`` (plain loops in double precision, see
the header there for the equations and the passages of the pages they follow).
This module only builds that file with gcc, loads it with ctypes and marshals
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at a deliberately broken copy of the oracle.
_SO_OVERRIDE = os.environ.get("GDN_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into liboracle.so (gcc -O2, OpenMP, no BLAS)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        path = _SO_OVERRIDE or _SO
        if not _SO_OVERRIDE and not os.path.exists(_SO):
            build(force=True)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn_oracle_scan.argtypes = [ctypes.c_int] * 6 + [dp] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp]
        lib.gdn_oracle_scan.restype = ctypes.c_int
        lib.gdn_oracle_scan_bwd.argtypes = [ctypes.c_int] * 6 + [dp] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [dp] * 8
        lib.gdn_oracle_scan_bwd.restype = ctypes.c_int
        lib.gdn_oracle_max_threads.argtypes = []
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def scan(q, k, v, beta, alpha, S0=None, *, eps: float = 1e-6,
         gates_are_logits: bool = False, normalize_keys: bool = True, reverse: bool = False):
    """Run the whole scan in fp64.

    q, k: [B,F,N,H,Dk]; v: [B,F,N,H,Dv]; beta: [B,F,N,H]; alpha: [B,F,H];
    S0: [B,H,Dv,Dk] or None (zeros).  Any real dtype; values are upcast
    exactly to float64.  normalize_keys=False uses the keys as given;
    reverse=True walks the frames from last to first.
    Returns (o [B,F,N,H,Dv], S_final [B,H,Dv,Dk]) as float64 arrays.
    """
    q, k, v, beta, alpha = (_f64(x) for x in (q, k, v, beta, alpha))
    B, F, N, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:4] != (B, F, N, H):
        raise ValueError("q/k/v shapes disagree")
    if beta.shape != (B, F, N, H) or alpha.shape != (B, F, H):
        raise ValueError("beta/alpha shapes disagree")
    if S0 is not None:
        S0 = _f64(S0)
        if S0.shape != (B, H, Dv, Dk):
            raise ValueError("S0 shape disagrees")
    o = np.zeros((B, F, N, H, Dv), dtype=np.float64)
    S_final = np.zeros((B, H, Dv, Dk), dtype=np.float64)
    rc = _load().gdn_oracle_scan(B, H, F, N, Dk, Dv, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(beta), _ptr(alpha), _ptr(S0), float(eps),
                                 int(bool(gates_are_logits)), int(bool(normalize_keys)),
                                 int(bool(reverse)), _ptr(o), _ptr(S_final))
    if rc != 0:
        raise RuntimeError("gdn_oracle_scan failed with code %d" % rc)
    return o, S_final


def scan_bwd(q, k, v, beta, alpha, S0, dO, dS_final=None, *, eps: float = 1e-6,
             gates_are_logits: bool = False, normalize_keys: bool = True, reverse: bool = False):
    """Gradients of the scan in fp64: given dO = dL/dO and dS_final = dL/dS_final
    (None: zeros), returns (dq, dk, dv, dbeta, dalpha, dS0), each in the
    layout of its input (dbeta, dalpha are logit gradients with
    gates_are_logits; dS0 is returned even when S0 is None)."""
    q, k, v, beta, alpha, dO = (_f64(x) for x in (q, k, v, beta, alpha, dO))
    B, F, N, H, Dk = q.shape
    Dv = v.shape[-1]
    if dO.shape != (B, F, N, H, Dv):
        raise ValueError("dO shape disagrees")
    S0 = None if S0 is None else _f64(S0)
    dS_final = None if dS_final is None else _f64(dS_final)
    outs = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(beta),
            np.zeros_like(alpha), np.zeros((B, H, Dv, Dk))]
    rc = _load().gdn_oracle_scan_bwd(B, H, F, N, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                     _ptr(alpha), _ptr(S0), float(eps), int(bool(gates_are_logits)),
                                     int(bool(normalize_keys)), int(bool(reverse)), _ptr(dO),
                                     _ptr(dS_final), *[_ptr(x) for x in outs])
    if rc != 0:
        raise RuntimeError("gdn_oracle_scan_bwd failed with code %d" % rc)
    return tuple(outs)


if __name__ == "__main__":  # pragma: no cover - manual rebuild helper
    print(build(force=True), file=sys.stderr)
