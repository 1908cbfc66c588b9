"""Python entry points with the same names as the C ABI (argument marshalling only)."""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import (KDA_BF16, KDA_FP32, KDA_GATE_BOUNDED, KDA_GATE_NONE, KDA_GATE_SOFTPLUS,
                   KdaFwdArgs, load, strerror)

_GATES = {None: KDA_GATE_NONE, "softplus": KDA_GATE_SOFTPLUS, "bounded": KDA_GATE_BOUNDED}

_IO = {torch.bfloat16: KDA_BF16, torch.float32: KDA_FP32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KdaFwdPlan:
    """Validated arguments for repeated kda_fwd calls on the same tensors.

    q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV] (all bf16 or all fp32, on one
    HIP device); cu_seqlens int64 [N+1] on the device (then B == 1) or None; initial_state fp32
    [N,HV,K,V] or None. Outputs o (io dtype, like v) and final_state (fp32, or None) and the
    workspace are allocated once through torch and reused by every call().

    Pre-stage, done inside the kernels: use_qk_l2norm divides each token's q and k by
    sqrt(sum of squares + 1e-6); use_beta_sigmoid takes beta as logits; gate "softplus"
    (g <- -exp(A_log) softplus(g + dt_bias)) or "bounded" (g <- gate_lower_bound *
    sigmoid(exp(A_log) (g + dt_bias))) takes g as the raw gate input, with A_log fp32 [HV] and
    dt_bias fp32 [HV, K] or None.
    """

    def __init__(self, q, k, v, g, beta, scale=None, cu_seqlens=None, initial_state=None,
                 output_final_state=True, workspace=None, o=None, final_state=None, chunk=0,
                 use_qk_l2norm=False, use_beta_sigmoid=False, gate=None, A_log=None,
                 dt_bias=None, gate_lower_bound=-5.0):
        self.lib = load()
        if q.dtype not in _IO:
            raise TypeError(f"unsupported io dtype {q.dtype} (bf16 or fp32)")
        dev = q.device
        if dev.type != "cuda":
            raise ValueError("inputs must be on a HIP device")
        B, T, H, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        dt = q.dtype
        _check(q, "q", dt, (B, T, H, K), dev)
        _check(k, "k", dt, (B, T, H, K), dev)
        _check(v, "v", dt, (B, T, HV, V), dev)
        _check(g, "g", dt, (B, T, HV, K), dev)
        _check(beta, "beta", dt, (B, T, HV), dev)
        if cu_seqlens is not None:
            if cu_seqlens.dtype != torch.int64 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
                raise ValueError("cu_seqlens must be a 1-D int64 tensor on the inputs' device")
            N = cu_seqlens.numel() - 1
        else:
            N = B
        if initial_state is not None:
            _check(initial_state, "initial_state", torch.float32, (N, HV, K, V), dev)
        self.o = torch.empty_like(v) if o is None else o
        _check(self.o, "o", dt, (B, T, HV, V), dev)
        if output_final_state:
            self.final_state = (torch.empty(N, HV, K, V, dtype=torch.float32, device=dev)
                                if final_state is None else final_state)
            _check(self.final_state, "final_state", torch.float32, (N, HV, K, V), dev)
        else:
            self.final_state = None
        a = KdaFwdArgs()
        a.B, a.T, a.N, a.H, a.HV, a.K, a.V, a.io = B, T, N, H, HV, K, V, _IO[dt]
        a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
        a.scale = float("nan") if scale is None else float(scale)
        a.cu_seqlens = _ptr(cu_seqlens)
        a.initial_state = _ptr(initial_state)
        a.o = _ptr(self.o)
        a.final_state = _ptr(self.final_state)
        a.chunk = int(chunk)
        if gate not in _GATES:
            raise ValueError(f"gate must be None, 'softplus' or 'bounded' (got {gate!r})")
        a.qk_l2norm = int(bool(use_qk_l2norm))
        a.beta_sigmoid = int(bool(use_beta_sigmoid))
        a.gate = _GATES[gate]
        a.gate_lower_bound = float(gate_lower_bound)
        if gate is not None:
            if A_log is None:
                raise ValueError("a gate needs A_log")
            _check(A_log, "A_log", torch.float32, (HV,), dev)
            if dt_bias is not None:
                _check(dt_bias, "dt_bias", torch.float32, (HV, K), dev)
            a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
        self.args = a
        self._keep = (q, k, v, g, beta, cu_seqlens, initial_state, A_log, dt_bias)
        need = int(self.lib.kda_fwd_workspace_bytes(ctypes.byref(a)))
        # 0 means "rejected", except for the token recurrence (chunk 1, which chunk 0 selects
        # for a dense batch of at most 16 tokens per sequence): it needs no workspace, and its
        # shape errors surface as the call's status
        recurrent = int(chunk) == 1 or (int(chunk) == 0 and cu_seqlens is None and T <= 16)
        if need == 0 and B * T > 0 and not recurrent:
            raise ValueError("unsupported shapes or chunk (K, V in {64, 128}; HV % H == 0; "
                             "chunk 1, 16, or 32 with bf16 io)")
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        elif workspace.numel() < need:
            raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
        self.workspace = workspace
        self.ws_bytes = workspace.numel()
        self.device = dev

    def _run(self, fn, name, stream):
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        st = fn(ctypes.byref(self.args), ctypes.c_void_p(self.workspace.data_ptr()),
                self.ws_bytes, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"{name} failed: {strerror(st)} ({st})")

    def __call__(self, stream=None):
        """Enqueue the forward on `stream` (default: torch's current stream)."""
        self._run(self.lib.kda_fwd, "kda_fwd", stream)
        return self.o, self.final_state

    def prepare(self, stream=None):
        """Enqueue only the prepare kernel (kda_fwd_prepare)."""
        self._run(self.lib.kda_fwd_prepare, "kda_fwd_prepare", stream)

    def state(self, stream=None):
        """Enqueue only the state kernel (kda_fwd_state); returns (o, final_state)."""
        self._run(self.lib.kda_fwd_state, "kda_fwd_state", stream)
        return self.o, self.final_state


class KdaBwdPlan:
    """Validated arguments for repeated kda_bwd calls: gradients of the forward with respect to
    q, k, v, g, beta, initial_state and (with a gate) A_log, dt_bias, from d_o (like v) and dht
    (fp32 [N,HV,K,V] or None).

    Inputs and pre-stage keywords as for KdaFwdPlan (with the pre-stage on, q, k, g, beta are
    the raw inputs and their gradients are the raw ones). Outputs, allocated once through
    torch and reused by every call(), all fp32: dq, dk [B,T,H,K]; dv [B,T,HV,V]; dg [B,T,HV,K];
    dbeta [B,T,HV]; dh0 [N,HV,K,V] (when want_dh0); dA_log [HV] and ddt_bias [HV,K] (with a
    gate).
    """

    def __init__(self, q, k, v, g, beta, d_o, dht=None, scale=None, cu_seqlens=None,
                 initial_state=None, want_dh0=True, workspace=None, use_qk_l2norm=False,
                 use_beta_sigmoid=False, gate=None, A_log=None, dt_bias=None,
                 gate_lower_bound=-5.0):
        self.lib = load()
        if q.dtype not in _IO:
            raise TypeError(f"unsupported io dtype {q.dtype} (bf16 or fp32)")
        dev = q.device
        if dev.type != "cuda":
            raise ValueError("inputs must be on a HIP device")
        B, T, H, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        dt = q.dtype
        for t, name, shape in ((q, "q", (B, T, H, K)), (k, "k", (B, T, H, K)),
                               (v, "v", (B, T, HV, V)), (g, "g", (B, T, HV, K)),
                               (beta, "beta", (B, T, HV)), (d_o, "d_o", (B, T, HV, V))):
            _check(t, name, dt, shape, dev)
        if cu_seqlens is not None:
            if cu_seqlens.dtype != torch.int64 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
                raise ValueError("cu_seqlens must be a 1-D int64 tensor on the inputs' device")
            N = cu_seqlens.numel() - 1
        else:
            N = B
        if initial_state is not None:
            _check(initial_state, "initial_state", torch.float32, (N, HV, K, V), dev)
        if dht is not None:
            _check(dht, "dht", torch.float32, (N, HV, K, V), dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.dq = torch.empty(B, T, H, K, **f32)
        self.dk = torch.empty(B, T, H, K, **f32)
        self.dv = torch.empty(B, T, HV, V, **f32)
        self.dg = torch.empty(B, T, HV, K, **f32)
        self.dbeta = torch.empty(B, T, HV, **f32)
        self.dh0 = torch.empty(N, HV, K, V, **f32) if want_dh0 else None
        if gate not in _GATES:
            raise ValueError(f"gate must be None, 'softplus' or 'bounded' (got {gate!r})")
        self.dA_log = torch.empty(HV, **f32) if gate is not None else None
        self.ddt_bias = torch.empty(HV, K, **f32) if gate is not None else None
        a = KdaFwdArgs()
        a.B, a.T, a.N, a.H, a.HV, a.K, a.V, a.io = B, T, N, H, HV, K, V, _IO[dt]
        a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
        a.scale = float("nan") if scale is None else float(scale)
        a.cu_seqlens = _ptr(cu_seqlens)
        a.initial_state = _ptr(initial_state)
        a.chunk = 16
        a.qk_l2norm = int(bool(use_qk_l2norm))
        a.beta_sigmoid = int(bool(use_beta_sigmoid))
        a.gate = _GATES[gate]
        a.gate_lower_bound = float(gate_lower_bound)
        if gate is not None:
            if A_log is None:
                raise ValueError("a gate needs A_log")
            _check(A_log, "A_log", torch.float32, (HV,), dev)
            if dt_bias is not None:
                _check(dt_bias, "dt_bias", torch.float32, (HV, K), dev)
            a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
        self.args = a
        self._keep = (q, k, v, g, beta, d_o, dht, cu_seqlens, initial_state, A_log, dt_bias)
        self._ptrs = [_ptr(d_o), _ptr(dht)]
        self._outs = [_ptr(x) for x in (self.dq, self.dk, self.dv, self.dg, self.dbeta,
                                        self.dh0, self.dA_log, self.ddt_bias)]
        need = int(self.lib.kda_bwd_workspace_bytes(ctypes.byref(a)))
        if need == 0:
            raise ValueError("unsupported shapes (K, V in {64, 128}; HV % H == 0)")
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        elif workspace.numel() < need:
            raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
        self.workspace = workspace
        self.ws_bytes = workspace.numel()
        self.device = dev

    def __call__(self, stream=None):
        """Enqueue the backward on `stream` (default: torch's current stream); returns
        (dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        st = self.lib.kda_bwd(ctypes.byref(self.args), *self._ptrs,
                              ctypes.c_void_p(self.workspace.data_ptr()), self.ws_bytes,
                              *self._outs, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"kda_bwd failed: {strerror(st)} ({st})")
        return (self.dq, self.dk, self.dv, self.dg, self.dbeta, self.dh0, self.dA_log,
                self.ddt_bias)


def kda_bwd(q, k, v, g, beta, d_o, dht=None, scale=None, cu_seqlens=None, initial_state=None,
            want_dh0=True, **prestage):
    """KDA backward. Returns fp32 (dq, dk, dv, dg, dbeta, dh0 or None, dA_log or None,
    ddt_bias or None); see KdaBwdPlan for shapes and the pre-stage keywords."""
    return KdaBwdPlan(q, k, v, g, beta, d_o, dht, scale, cu_seqlens, initial_state,
                      want_dh0, **prestage)()


def kda_fwd(q, k, v, g, beta, scale=None, cu_seqlens=None, initial_state=None,
            output_final_state=True, workspace=None, chunk=0, **prestage):
    """KDA forward. Returns (o, final_state or None); see KdaFwdPlan for shapes and the
    pre-stage keywords (use_qk_l2norm, use_beta_sigmoid, gate, A_log, dt_bias,
    gate_lower_bound)."""
    plan = KdaFwdPlan(q, k, v, g, beta, scale, cu_seqlens, initial_state, output_final_state,
                      workspace, chunk=chunk, **prestage)
    return plan()


def workspace_bytes(B, T, N, H, HV, K, V, io=KDA_BF16, chunk=0) -> int:
    """Workspace bytes kda_fwd needs for these shapes (0 if unsupported)."""
    a = KdaFwdArgs()
    a.B, a.T, a.N, a.H, a.HV, a.K, a.V, a.io = B, T, N, H, HV, K, V, io
    a.chunk = chunk
    return int(load().kda_fwd_workspace_bytes(ctypes.byref(a)))
