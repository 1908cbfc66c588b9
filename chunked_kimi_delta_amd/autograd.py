"""torch.autograd integration: chunk_kda runs kda_fwd forward and kda_bwd backward (argument
marshalling only; both directions are the library's kernels)."""
from __future__ import annotations

import torch

from .api import kda_bwd, kda_fwd


class ChunkKDAFunction(torch.autograd.Function):
    """o, final_state = KDA(q, k, v, g, beta; initial_state), differentiable in q, k, v, g, beta,
    initial_state and (with a gate) A_log, dt_bias. Gradients come back in the dtype of each
    input (the kernels compute them in fp32)."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, A_log, dt_bias, scale, cu_seqlens,
                use_qk_l2norm, use_beta_sigmoid, gate, gate_lower_bound):
        pre = dict(use_qk_l2norm=use_qk_l2norm, use_beta_sigmoid=use_beta_sigmoid, gate=gate,
                   A_log=A_log, dt_bias=dt_bias, gate_lower_bound=gate_lower_bound)
        o, fin = kda_fwd(q, k, v, g, beta, scale=scale, cu_seqlens=cu_seqlens,
                         initial_state=initial_state, output_final_state=True, **pre)
        ctx.save_for_backward(q, k, v, g, beta, initial_state, A_log, dt_bias, cu_seqlens)
        ctx.scale = scale
        ctx.pre = dict(use_qk_l2norm=use_qk_l2norm, use_beta_sigmoid=use_beta_sigmoid, gate=gate,
                       gate_lower_bound=gate_lower_bound)
        return o, fin

    @staticmethod
    def backward(ctx, d_o, d_fin):
        q, k, v, g, beta, h0, A_log, dt_bias, cu = ctx.saved_tensors
        d_o = (torch.zeros_like(v) if d_o is None else d_o.to(v.dtype)).contiguous()
        dht = None if d_fin is None else d_fin.float().contiguous()
        dq, dk, dv, dg, db, dh0, dA, ddt = kda_bwd(
            q, k, v, g, beta, d_o, dht, scale=ctx.scale, cu_seqlens=cu, initial_state=h0,
            want_dh0=h0 is not None, A_log=A_log, dt_bias=dt_bias, **ctx.pre)
        cast = lambda x, ref: None if x is None or ref is None else x.to(ref.dtype)
        return (cast(dq, q), cast(dk, k), cast(dv, v), cast(dg, g), cast(db, beta),
                cast(dh0, h0), cast(dA, A_log), cast(ddt, dt_bias),
                None, None, None, None, None, None)


def chunk_kda(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
              use_qk_l2norm=False, use_beta_sigmoid=False, gate=None, A_log=None, dt_bias=None,
              gate_lower_bound=-5.0):
    """Differentiable KDA forward; returns (o, final_state). Shapes as KdaFwdPlan; every
    tensor argument may require grad (cu_seqlens excepted). The forward uses the library's
    default chunk; the backward always uses 16-token chunks."""
    return ChunkKDAFunction.apply(q, k, v, g, beta, initial_state, A_log, dt_bias, scale,
                                  cu_seqlens, use_qk_l2norm, use_beta_sigmoid, gate,
                                  gate_lower_bound)
