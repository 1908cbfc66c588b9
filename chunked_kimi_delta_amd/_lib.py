"""ctypes view of libkda_fwd's C ABI (include/kda_fwd.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libkda_fwd.so"

(KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP,
 KDA_ERR_NOALLOC_TOO_LARGE) = range(6)
KDA_NOALLOC_WORKSPACE_BYTES = 128 << 20
KDA_BF16, KDA_FP32 = 0, 1
KDA_GATE_NONE, KDA_GATE_SOFTPLUS, KDA_GATE_BOUNDED = 0, 1, 2


class KdaFwdArgs(ctypes.Structure):
    """Mirror of kda_fwd_args."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("N", ctypes.c_int32),
        ("H", ctypes.c_int32), ("HV", ctypes.c_int32), ("K", ctypes.c_int32),
        ("V", ctypes.c_int32), ("io", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("cu_seqlens", ctypes.c_void_p), ("initial_state", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("chunk", ctypes.c_int32),
        ("qk_l2norm", ctypes.c_int32), ("beta_sigmoid", ctypes.c_int32),
        ("gate", ctypes.c_int32), ("gate_lower_bound", ctypes.c_float),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
    ]


def library_path() -> str:
    return os.environ.get("KDA_FWD_LIB", os.path.join(HERE, LIB_NAME))


_lib = None


def load():
    """Load libkda_fwd.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build the HIP library first "
            "(python -m chunked_kimi_delta_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.kda_fwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaFwdArgs)]
    lib.kda_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_fwd.argtypes = [ctypes.POINTER(KdaFwdArgs), ctypes.c_void_p, ctypes.c_size_t,
                            ctypes.c_void_p]
    lib.kda_fwd.restype = ctypes.c_int
    for name in ("kda_fwd_prepare", "kda_fwd_state"):
        f = getattr(lib, name)
        f.argtypes = lib.kda_fwd.argtypes
        f.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = [ctypes.POINTER(KdaFwdArgs), ctypes.c_void_p]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_bwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaFwdArgs)]
    lib.kda_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_bwd.argtypes = ([ctypes.POINTER(KdaFwdArgs), ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_void_p] * 9)
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_strerror.argtypes = [ctypes.c_int]
    lib.kda_strerror.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().kda_strerror(status).decode()
