"""fp64 CPU oracle for causal grouped-query attention (test infrastructure).

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package. It shares no code with the HIP library and is never a fallback for it.

The arithmetic lives in ``cgqa_oracle.c`` (plain loops, double precision, the whole
score matrix written out per head, as the naive kernels of the page "A transformer in
PTX", section "Flash attention", do). This module only marshals numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path):
    """Load an oracle shared library (the default one, or a test's planted-mistake build)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double, i]
    lib.oracle_attn_fwd.restype = i
    lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                    i, i, i, i, i, ctypes.c_double, i]
    lib.oracle_attn_bwd.restype = i
    lib.oracle_bf16_to_f64.argtypes = [ctypes.POINTER(ctypes.c_uint16), dp, ctypes.c_long]
    lib.oracle_bf16_to_f64.restype = i
    lib.oracle_default_threads.argtypes = []
    lib.oracle_default_threads.restype = i
    return lib


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    src = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(src.shape, dtype=np.float64)
    rc = _load().oracle_bf16_to_f64(src.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                    _dptr(out), src.size)
    if rc != 0:
        raise ValueError(f"oracle_bf16_to_f64 failed ({rc})")
    return out


def _shapes(q, k):
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q and k must be [B, T, H, d]")
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, T, Hkv, d):
        raise ValueError(f"k shape {k.shape} does not match q shape {q.shape}")
    return B, T, Hq, Hkv, d


def attn_fwd(q, k, v, scale, threads=0, lib=None):
    """Returns (o [B,T,Hq,d], lse [B,Hq,T]) in float64 for fp64 inputs."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, Hkv, d = _shapes(q, k)
    if v.shape != k.shape:
        raise ValueError("v must have k's shape")
    o = np.zeros((B, T, Hq, d))
    lse = np.zeros((B, Hq, T))
    rc = (lib or _load()).oracle_attn_fwd(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse),
                                 B, T, Hq, Hkv, d, float(scale), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd failed ({rc})")
    return o, lse


def attn_bwd(q, k, v, do, scale, threads=0, lib=None):
    """Returns dict(o, lse, delta, dq, dk, dv), all float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, T, Hq, Hkv, d = _shapes(q, k)
    if v.shape != k.shape or do.shape != q.shape:
        raise ValueError("v must have k's shape and dO q's shape")
    out = dict(o=np.zeros((B, T, Hq, d)), lse=np.zeros((B, Hq, T)), delta=np.zeros((B, Hq, T)),
               dq=np.zeros((B, T, Hq, d)), dk=np.zeros((B, T, Hkv, d)),
               dv=np.zeros((B, T, Hkv, d)))
    rc = (lib or _load()).oracle_attn_bwd(_dptr(q), _dptr(k), _dptr(v), _dptr(do),
                                 _dptr(out["o"]), _dptr(out["lse"]), _dptr(out["delta"]),
                                 _dptr(out["dq"]), _dptr(out["dk"]), _dptr(out["dv"]),
                                 B, T, Hq, Hkv, d, float(scale), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd failed ({rc})")
    return out
