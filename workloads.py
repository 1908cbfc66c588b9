"""Seeded synthetic inputs for the chunked KDA forward.

This module only *draws* inputs: it holds none of the method's arithmetic, so both the
CPU oracle and the HIP path can be fed from it without sharing any computation.

Workloads mirror the shapes of the pages' kernels (head dim 128, chunk 16, grouped value
heads, packed variable-length batches) and the five named configurations below. Every tensor
is drawn in fp32 on the CPU from ``torch.Generator().manual_seed(seed)`` in a fixed order
(lengths, q, k, v, g, beta, initial state), transformed in fp32, then cast to the io dtype.
The oracle reads the cast values (bf16 -> fp32 is exact), so both sides see bit-identical
inputs.

Distributions (second parameter of N(.,.) is a standard deviation):
  q, k   ~ N(0,1), then per-token L2 normalisation x * rsqrt(sum x^2 + 1e-6)
           (the normalisation used by the pages' pre-stage, "手撕KDA" CPU reference)
  v      ~ N(0,1)
  g      = log(u), u ~ U(lo, hi) per token, per value head, per key dim (natural-log decay)
  beta   = sigmoid(N(0, beta_std))
  h0     ~ N(0, h0_std) in fp32 when requested
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

L2_EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    dtype: str                     # "bf16" or "fp32" (io dtype of q, k, v, g, beta, o)
    g_lo: float = 0.9
    g_hi: float = 0.999
    beta_std: float = 1.0
    h0_std: Optional[float] = None  # None -> no initial state
    n_seqs: Optional[int] = None    # varlen: number of packed sequences (B must be 1)
    len_lo: int = 0
    len_hi: int = 0
    lengths: Optional[tuple] = None  # explicit varlen lengths (overrides the random draw)

    @property
    def G(self) -> int:
        return self.HV // self.H


# The five named workloads. "tiny_fp32" is the small case the oracle finishes instantly;
# "h16_t4096" is the throughput workload.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, T=64, H=1, HV=1, K=64, V=64, dtype="fp32"),
    "h16_t4096": Workload("h16_t4096", B=1, T=4096, H=16, HV=16, K=128, V=128, dtype="bf16"),
    # the same in fp32 io (the fp32 mode at the benchmark's size)
    "h16_t4096_fp32": Workload("h16_t4096_fp32", B=1, T=4096, H=16, HV=16, K=128, V=128,
                               dtype="fp32"),
    "varlen8_h32": Workload("varlen8_h32", B=1, T=0, H=32, HV=32, K=128, V=128, dtype="bf16",
                            h0_std=0.1, n_seqs=8, len_lo=256, len_hi=8192),
    "gva_b4_t8192": Workload("gva_b4_t8192", B=4, T=8192, H=16, HV=32, K=128, V=128,
                             dtype="bf16"),
    "long_t131072": Workload("long_t131072", B=1, T=131072, H=32, HV=32, K=128, V=128,
                             dtype="bf16", g_lo=0.5, g_hi=0.9999, beta_std=2.0),
    # one decoding step of a batch: 64 sequences, one new token each, carried state
    "decode_b64_h32": Workload("decode_b64_h32", B=64, T=1, H=32, HV=32, K=128, V=128,
                               dtype="bf16", h0_std=0.1),
}


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit fields (edge cases, small parity shapes)."""
    base = dict(B=1, T=64, H=1, HV=1, K=64, V=64, dtype="bf16")
    base.update(kw)
    return Workload(name, **base)


def _torch_dtype(d: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[d]


def draw_lengths(w: Workload, gen: torch.Generator) -> list:
    """Varlen lengths: uniform integers in [len_lo, len_hi], each rounded to the nearest
    multiple of 16 (ties away from zero)."""
    if w.lengths is not None:
        return list(w.lengths)
    raw = torch.randint(w.len_lo, w.len_hi + 1, (w.n_seqs,), generator=gen)
    return [int(16 * math.floor(x / 16 + 0.5)) for x in raw.tolist()]


def _l2n(x: torch.Tensor) -> torch.Tensor:
    return x * torch.rsqrt((x * x).sum(-1, keepdim=True) + L2_EPS)


@dataclasses.dataclass
class Inputs:
    w: Workload
    q: torch.Tensor                 # [B, T, H, K]  io dtype, CPU
    k: torch.Tensor                 # [B, T, H, K]
    v: torch.Tensor                 # [B, T, HV, V]
    g: torch.Tensor                 # [B, T, HV, K]
    beta: torch.Tensor              # [B, T, HV]
    h0: Optional[torch.Tensor]      # [N, HV, K, V] fp32 or None
    cu_seqlens: Optional[torch.Tensor]  # int64 [N+1] or None
    scale: float

    @property
    def N(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def T_total(self) -> int:
        return self.q.shape[0] * self.q.shape[1]

    def seq_bounds(self):
        """[(bos, eos)] over the packed token axis (B*T tokens)."""
        if self.cu_seqlens is None:
            T = self.q.shape[1]
            return [(b * T, (b + 1) * T) for b in range(self.q.shape[0])]
        c = self.cu_seqlens.tolist()
        return [(c[i], c[i + 1]) for i in range(len(c) - 1)]


def make_inputs(w: Workload, seed: int = 0, g_override=None, beta_override=None) -> Inputs:
    """Draw one seeded input set for workload ``w`` (CPU tensors)."""
    gen = torch.Generator().manual_seed(seed)
    cu = None
    B, T = w.B, w.T
    if w.n_seqs is not None or w.lengths is not None:
        lens = draw_lengths(w, gen)
        B, T = 1, int(sum(lens))
        cu = torch.tensor([0] + list(torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0)),
                          dtype=torch.int64)
    dt = _torch_dtype(w.dtype)
    q = _l2n(torch.randn(B, T, w.H, w.K, generator=gen)).to(dt)
    k = _l2n(torch.randn(B, T, w.H, w.K, generator=gen)).to(dt)
    v = torch.randn(B, T, w.HV, w.V, generator=gen).to(dt)
    u = torch.rand(B, T, w.HV, w.K, generator=gen) * (w.g_hi - w.g_lo) + w.g_lo
    g = torch.log(u)
    if g_override is not None:
        g = torch.full_like(g, float(g_override))
    g = g.to(dt)
    beta = torch.sigmoid(torch.randn(B, T, w.HV, generator=gen) * w.beta_std)
    if beta_override is not None:
        beta = torch.full_like(beta, float(beta_override))
    beta = beta.to(dt)
    N = B if cu is None else cu.numel() - 1
    h0 = None
    if w.h0_std is not None:
        h0 = torch.randn(N, w.HV, w.K, w.V, generator=gen) * w.h0_std
    return Inputs(w, q, k, v, g, beta, h0, cu, scale=w.K ** -0.5)


@dataclasses.dataclass
class RawInputs:
    """Raw projections for the fused pre-stage: q, k not normalised, g the raw gate input,
    beta logits, plus the per-value-head gate parameters (fp32)."""
    inp: Inputs                     # q, k, g, beta raw (io dtype); v, h0, cu_seqlens as usual
    A_log: torch.Tensor             # [HV] fp32
    dt_bias: torch.Tensor           # [HV, K] fp32


def make_raw_inputs(w: Workload, seed: int = 0, qk_std: float = 2.0, g_mean: float = -1.0,
                    A_lo: float = 0.5, A_hi: float = 2.0, dt_std: float = 0.5) -> RawInputs:
    """Draw one seeded raw input set (CPU tensors) in the order lengths, q, k, v, g_raw,
    beta_raw, h0, A_log, dt_bias:
      q, k ~ N(0, qk_std) (not normalised)     v ~ N(0, 1)
      g_raw ~ N(g_mean, 1)                      beta_raw ~ N(0, beta_std)
      A_log = log U(A_lo, A_hi) per value head  dt_bias ~ N(0, dt_std) per value head and dim
    With the softplus gate the log decay per token stays above about -2 A_hi * 1.5, so any 16
    consecutive tokens sum well above -88 (the chunked kernels' range)."""
    gen = torch.Generator().manual_seed(seed)
    cu = None
    B, T = w.B, w.T
    if w.n_seqs is not None or w.lengths is not None:
        lens = draw_lengths(w, gen)
        B, T = 1, int(sum(lens))
        cu = torch.tensor([0] + list(torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0)),
                          dtype=torch.int64)
    dt = _torch_dtype(w.dtype)
    q = (torch.randn(B, T, w.H, w.K, generator=gen) * qk_std).to(dt)
    k = (torch.randn(B, T, w.H, w.K, generator=gen) * qk_std).to(dt)
    v = torch.randn(B, T, w.HV, w.V, generator=gen).to(dt)
    g = (torch.randn(B, T, w.HV, w.K, generator=gen) + g_mean).to(dt)
    beta = (torch.randn(B, T, w.HV, generator=gen) * w.beta_std).to(dt)
    N = B if cu is None else cu.numel() - 1
    h0 = None
    if w.h0_std is not None:
        h0 = torch.randn(N, w.HV, w.K, w.V, generator=gen) * w.h0_std
    A_log = torch.log(torch.rand(w.HV, generator=gen) * (A_hi - A_lo) + A_lo)
    dt_bias = torch.randn(w.HV, w.K, generator=gen) * dt_std
    return RawInputs(Inputs(w, q, k, v, g, beta, h0, cu, scale=w.K ** -0.5), A_log, dt_bias)


@dataclasses.dataclass
class Grads:
    d_o: torch.Tensor               # [B, T, HV, V] io dtype, CPU: gradient of o
    dht: Optional[torch.Tensor]     # [N, HV, K, V] fp32 or None: gradient of the final state


def make_grads(inp: Inputs, seed: int = 0, dht_std: Optional[float] = 1.0) -> Grads:
    """Seeded incoming gradients for a backward pass over ``inp``: d_o ~ N(0, 1) in the io
    dtype, dht ~ N(0, dht_std) in fp32 (None when dht_std is None)."""
    gen = torch.Generator().manual_seed(10_000 + seed)
    B, T, HV, V = inp.v.shape
    K = inp.q.shape[3]
    d_o = torch.randn(B, T, HV, V, generator=gen).to(inp.v.dtype)
    dht = (None if dht_std is None
           else torch.randn(inp.N, HV, K, V, generator=gen) * dht_std)
    return Grads(d_o, dht)


def as_f32_numpy(x: Optional[torch.Tensor]):
    """Exact fp32 copy of an io-dtype tensor (bf16 -> fp32 is exact) as a numpy array."""
    if x is None:
        return None
    return x.float().contiguous().numpy()
