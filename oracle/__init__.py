"""Double-precision CPU oracle for causal GQA attention with RoPE (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  The arithmetic lives
in ne_oracle.c (see its header for the passages it follows); this module only
marshals numpy float64 arrays.

Layouts: q, o, dO, dq [B,T,Hq,D]; k, v, dk, dv [B,T,Hkv,D]; lse [B,Hq,T].
"""
import ctypes

import numpy as np

from . import build as _build
from .decode import decode_fwd, rope_rows  # noqa: F401  (numpy oracle of the cached-decode workload)
from .qkv import qkv_rope_proj  # noqa: F401  (numpy oracle of the QKV projection with RoPE epilogue)

_lib = None


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.ne_oracle_fwd.argtypes = [P, P, P, P, P, i, i, i, i, i, ctypes.c_double, i]
    lib.ne_oracle_fwd.restype = i
    lib.ne_oracle_bwd.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, ctypes.c_double, i]
    lib.ne_oracle_bwd.restype = i
    lib.ne_oracle_bwd_given_o.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, ctypes.c_double, i]
    lib.ne_oracle_bwd_given_o.restype = i
    lib.ne_oracle_fwd_w.argtypes = [P, P, P, P, P, i, i, i, i, i, ctypes.c_double, i, i]
    lib.ne_oracle_fwd_w.restype = i
    lib.ne_oracle_bwd_w.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, ctypes.c_double, i, i]
    lib.ne_oracle_bwd_w.restype = i
    lib.ne_oracle_bwd_given_o_w.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, ctypes.c_double, i, i]
    lib.ne_oracle_bwd_given_o_w.restype = i
    d = ctypes.c_double
    lib.ne_oracle_fwd_x.argtypes = [P, P, P, P, P, i, i, i, i, i, d, i, i, d, d, i, i]
    lib.ne_oracle_fwd_x.restype = i
    lib.ne_oracle_bwd_x.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, d, i, i, d, d, i, i]
    lib.ne_oracle_bwd_x.restype = i
    lib.ne_oracle_rope.argtypes = [P, P, i, i, i, i, ctypes.c_double, i, i]
    lib.ne_oracle_rope.restype = i
    lib.ne_oracle_max_threads.argtypes = []
    lib.ne_oracle_max_threads.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _bind(_build.build(force=False))
    return _lib


class use_library:
    """Temporarily route this module's calls to another build of the oracle source
    (the mutation tests compile deliberately broken copies and check that the pins fail)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q, k):
    B, T, Hq, D = q.shape
    Bk, Tk, Hkv, Dk = k.shape
    if (Bk, Tk, Dk) != (B, T, D):
        raise ValueError(f"q {q.shape} and k {k.shape} disagree")
    return B, T, Hq, Hkv, D


def _qk(qk_norm):
    """qk_norm: None (off) or (gain, eps)."""
    if qk_norm is None:
        return 0, 0.0, 0.0
    gain, eps = qk_norm
    return 1, float(gain), float(eps)


def fwd(q, k, v, rope_base, nthreads=0, window=0, qk_norm=None, half_split=False):
    """Return (o, lse) in float64.  window W > 0: query i sees keys i-W+1 .. i.
    qk_norm (gain, eps): every row of q and k becomes gain * x / sqrt(mean(x^2) + eps) first.
    half_split: the rotation pairs element i with element i + D/2 instead of (2i, 2i+1)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, Hkv, D = _dims(q, k)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    rc = _load().ne_oracle_fwd_x(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D,
                                 float(rope_base), int(window), *_qk(qk_norm), int(bool(half_split)), int(nthreads))
    if rc:
        raise ValueError(f"ne_oracle_fwd rejected the arguments (rc={rc})")
    return o, lse


def _bwd(q, k, v, o, dO, rope_base, nthreads, window, qk_norm, half_split):
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, T, Hq, Hkv, D = _dims(q, k)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    optr = None
    if o is not None:
        o = _f64(o)
        optr = _ptr(o)
    rc = _load().ne_oracle_bwd_x(_ptr(q), _ptr(k), _ptr(v), optr, _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                                 B, T, Hq, Hkv, D, float(rope_base), int(window), *_qk(qk_norm), int(bool(half_split)),
                                 int(nthreads))
    if rc:
        raise ValueError(f"ne_oracle_bwd rejected the arguments (rc={rc})")
    return dq, dk, dv


def bwd(q, k, v, dO, rope_base, nthreads=0, window=0, qk_norm=None, half_split=False):
    """Return (dq, dk, dv) in float64: the exact gradients of sum(o * dO)."""
    return _bwd(q, k, v, None, dO, rope_base, nthreads, window, qk_norm, half_split)


def bwd_given_o(q, k, v, o, dO, rope_base, nthreads=0, window=0, qk_norm=None, half_split=False):
    """(dq, dk, dv) with Delta = rowsum(dO * o) from the given o (e.g. o stored in bf16)."""
    return _bwd(q, k, v, o, dO, rope_base, nthreads, window, qk_norm, half_split)


def rope(x, rope_base, inverse=False, half_split=False):
    """Rotate x [B,T,H,D] by R_t (or R_t^T when inverse); half_split: pairs (i, i + D/2)."""
    x = _f64(x)
    B, T, H, D = x.shape
    y = np.empty_like(x)
    rc = _load().ne_oracle_rope(_ptr(x), _ptr(y), B, T, H, D, float(rope_base), int(bool(inverse)),
                                int(bool(half_split)))
    if rc:
        raise ValueError("ne_oracle_rope rejected the arguments")
    return y


def max_threads():
    return int(_load().ne_oracle_max_threads())
