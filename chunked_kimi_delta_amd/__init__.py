"""Chunked Kimi Delta Attention (KDA) forward (and its backward) on AMD Instinct MI355X (gfx950).

The compute lives in libkda_fwd.so (hand-written HIP kernels behind the C ABI of
include/kda_fwd.h). This package is a thin ctypes binding: it marshals torch tensors' device
pointers and the current HIP stream into that ABI and nothing else. There is no fallback: if
the shared library is missing or cannot be loaded, every entry point raises.
"""
from .api import KdaBwdPlan, KdaFwdPlan, kda_bwd, kda_fwd, workspace_bytes  # noqa: F401
from .autograd import ChunkKDAFunction, chunk_kda  # noqa: F401
from ._lib import KDA_BF16, KDA_FP32, library_path, load  # noqa: F401

__all__ = ["kda_fwd", "KdaFwdPlan", "kda_bwd", "KdaBwdPlan", "chunk_kda", "ChunkKDAFunction",
           "workspace_bytes", "load", "library_path", "KDA_BF16", "KDA_FP32"]
