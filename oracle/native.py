"""ctypes binding of the C fp64 oracle (test infrastructure)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        f = lib.kda_oracle_fwd
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_double, P, P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int]
        f.restype = ctypes.c_int
        b = lib.kda_oracle_bwd
        b.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_double] + [P] * 14 + [ctypes.c_int]
        b.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def kda_oracle_c(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                 units=None, n_threads=None, want_o=True):
    """fp64 recurrence in C. Array shapes as recurrent.kda_recurrent. Inputs are converted to
    contiguous fp32 (they already hold bf16/fp32 values exactly). `units` = list of (s, j):
    only those units are computed (others stay zero). Returns (o [B,T,HV,V], final [N,HV,K,V])
    float64 (o is None when want_o is False)."""
    lib = _load()
    f32 = lambda x: None if x is None else np.ascontiguousarray(x, dtype=np.float32)
    q, k, v, g, beta = f32(q), f32(k), f32(v), f32(g), f32(beta)
    h0 = f32(initial_state)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if scale is None:
        scale = K ** -0.5
    if cu_seqlens is None:
        bounds = np.arange(B + 1, dtype=np.int64) * T
    else:
        bounds = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
    N = bounds.size - 1
    o = np.zeros((B, T, HV, V), np.float64) if want_o else None
    ht = np.zeros((N, HV, K, V), np.float64)
    if units is not None:
        u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = u.shape[0]
    else:
        u, n_units = None, 0
    nt = n_threads or default_threads()
    rc = lib.kda_oracle_fwd(N, _ptr(bounds), H, HV, K, V, float(scale), _ptr(q), _ptr(k),
                            _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
                            _ptr(u), n_units, nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with status {rc}")
    return o, ht


def kda_oracle_bwd_c(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                     do=None, dht=None, n_threads=None):
    """fp64 gradients in C (kda_oracle_bwd.c): the reverse token recurrence of
    backward.kda_backward_recurrent, over every unit. Shapes as there. Returns (dq, dk, dv, dg,
    dbeta, dh0) float64 (dh0 [N,HV,K,V])."""
    lib = _load()
    f32 = lambda x: None if x is None else np.ascontiguousarray(x, dtype=np.float32)
    q, k, v, g, beta = f32(q), f32(k), f32(v), f32(g), f32(beta)
    h0, do, dht = f32(initial_state), f32(do), f32(dht)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if scale is None:
        scale = K ** -0.5
    if cu_seqlens is None:
        bounds = np.arange(B + 1, dtype=np.int64) * T
    else:
        bounds = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
    N = bounds.size - 1
    dq = np.zeros((B, T, H, K), np.float64)
    dk = np.zeros((B, T, H, K), np.float64)
    dv = np.zeros((B, T, HV, V), np.float64)
    dg = np.zeros((B, T, HV, K), np.float64)
    db = np.zeros((B, T, HV), np.float64)
    dh0 = np.zeros((N, HV, K, V), np.float64)
    nt = n_threads or default_threads()
    rc = lib.kda_oracle_bwd(N, _ptr(bounds), H, HV, K, V, float(scale), _ptr(q), _ptr(k),
                            _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dh0), nt)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed with status {rc}")
    return dq, dk, dv, dg, db, dh0
