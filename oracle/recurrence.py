"""ORACLE (test infrastructure only): ctypes wrapper of the fp64 token recurrence.

See recurrence.c for the definition followed: the gated delta rule of
"Empowering Hybrid Attention Models on NPUs" (section 2.1, linear attention
with a per-head recurrent state), with a per-token log-decay g, alpha = exp(g),
scalar per head for GDN or per key channel for KDA, and varlen packing by
cu_seqlens as in the FLA graph-capture RFC (section "Fixed-capacity
execution").
"""

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        f = lib.oracle_gated_delta_fwd
        f.restype = ctypes.c_int
        f.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 6 +
                      [ctypes.c_int] * 5 + [ctypes.c_double] +
                      [ctypes.c_void_p] * 3 + [ctypes.c_int])
        lib.oracle_check_cu.restype = ctypes.c_int
        lib.oracle_check_cu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads():
    return _load().oracle_max_threads()


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def gated_delta_fwd(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0, *,
                    kda=False, with_state=True, nthreads=0):
    """fp64 token recurrence over a varlen batch.

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H] (GDN) or [T, H, dk] (KDA);
    beta: [T, H]; cu_seqlens: [N+1] int; h0: [N, H, dk, dv] or None.
    Returns (o [T, H, dv] fp64 with NaN on rows no sequence covers,
    ht [N, H, dk, dv] fp64 with NaN for zero-length sequences, or None).
    Raises ValueError for an invalid cu_seqlens.
    """
    lib = _load()
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and v.shape[:2] == (T, H)
    assert g.shape == ((T, H, dk) if kda else (T, H)), g.shape
    assert beta.shape == (T, H)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = len(cu) - 1
    if h0 is not None:
        h0 = np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
        assert h0.shape == (N, H, dk, dv)
    o = np.full((T, H, dv), np.nan)
    ht = np.full((N, H, dk, dv), np.nan) if with_state else None
    rc = lib.oracle_gated_delta_fwd(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(cu), N, T, H, dk, dv,
                                    float(scale), _ptr(h0), _ptr(o), _ptr(ht),
                                    int(nthreads))
    if rc > 0:
        raise ValueError(f"invalid cu_seqlens (code {rc})")
    if rc < 0:
        raise MemoryError("oracle scratch allocation failed")
    return o, ht
