"""ctypes front end of the fp64 C oracle (test infrastructure only).

The arithmetic lives in ``attn_oracle.c``; this module only widens inputs to
fp64, passes pointers and reshapes the outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")
_lib = None


def oracle_lib_path() -> str:
    return _LIB


def build_oracle(force: bool = True) -> str:
    """Compile attn_oracle.c into libattn_oracle.so with gcc (-O2, no fast-math:
    the oracle keeps IEEE fp64 semantics)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_oracle(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_attn_fwd
        f.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        f.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64,
                      ctypes.c_double, ctypes.c_int,
                      ctypes.POINTER(ctypes.c_int64), i64, ctypes.c_int]
        _lib = lib
    return _lib


def _as_f64(x) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor (any float dtype) to a
    contiguous fp64 numpy array.  Widening fp16/bf16/fp32 to fp64 is exact."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def attn_fwd_oracle(q, k, v, scale: float, causal: bool, rows=None,
                    nthreads: int | None = None):
    """Exact attention forward in fp64.

    q: (B, Sq, Hq, d); k, v: (B, Sk, Hkv, d).  Returns (o, lse):
      rows is None -> o (B, Sq, Hq, d), lse (B, Hq, Sq)
      rows given   -> rows are flat ids (b*Hq + h)*Sq + i; o (n, d), lse (n,)
    """
    qd, kd, vd = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Sq, Hq, d = qd.shape
    Bk, Sk, Hkv, dk = kd.shape
    if vd.shape != kd.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch between q, k, v")
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    dp = ctypes.POINTER(ctypes.c_double)
    if rows is None:
        o = np.empty((B, Sq, Hq, d), np.float64)
        lse = np.empty((B, Hq, Sq), np.float64)
        rows_p, n = None, 0
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = int(r.size)
        o = np.empty((n, d), np.float64)
        lse = np.empty((n,), np.float64)
        rows_p = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load().oracle_attn_fwd(
        qd.ctypes.data_as(dp), kd.ctypes.data_as(dp), vd.ctypes.data_as(dp),
        o.ctypes.data_as(dp), lse.ctypes.data_as(dp),
        B, Sq, Sk, Hq, Hkv, d, float(scale), int(bool(causal)),
        rows_p, n, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd failed with code {rc}")
    return o, lse
