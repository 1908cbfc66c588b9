"""fp64 token-by-token KDA recurrence: the definition of the forward (test infrastructure).

For one sequence and one value head j, with q/k head h = floor(j / G), G = HV / H, and a state
S in R^{K x V} (initial_state[s, j], or zeros), each token t does, in this order:

    S <- diag(exp(g[t, j, :])) S                 per-key-dimension decay (g is a natural log)
    r <- v[t, j, :] - S^T k[t, h, :]             delta-rule residual, read from the decayed S
    S <- S + beta[t, j] * k[t, h, :] r^T         rank-1 delta-rule write
    o[t, j, :] <- scale * S^T q[t, h, :]         read AFTER the write

and final_state[s, j] = S after the last token.

Source: "手撕KDA" ("KDA by hand"), section 1 (naive_chunk_kda). With a chunk of one token the
listing's in-chunk solve is A = beta, so w = beta*exp(g)*k and u = beta*v, and its chunk step
becomes exactly the four lines above; the Aqk diagonal it keeps is what makes the output read
after the write. Section 5 of the page names this recurrent form (fused_recurrent_kda) as the
cross-check of the chunked kernels. scale defaults to K**-0.5 and q/k are shared by the G value
heads of a group (the listing's repeat_interleave), as in the same section.
"""
from __future__ import annotations

import numpy as np


def _bounds(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    c = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    return [(c[i], c[i + 1]) for i in range(len(c) - 1)]


def kda_recurrent(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None):
    """Reference KDA forward by the token recurrence, in fp64.

    q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV]; initial_state [N,HV,K,V] or
    None; cu_seqlens int [N+1] (then B == 1) or None. Returns (o [B,T,HV,V], final [N,HV,K,V]),
    both float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    assert HV % H == 0
    G = HV // H
    if scale is None:
        scale = K ** -0.5
    bounds = _bounds(B, T, cu_seqlens)
    N = len(bounds)
    hq = np.arange(HV) // G                       # q/k head of each value head
    qf = q.reshape(B * T, H, K)
    kf = k.reshape(B * T, H, K)
    vf = v.reshape(B * T, HV, V)
    gf = g.reshape(B * T, HV, K)
    bf = beta.reshape(B * T, HV)
    o = np.zeros((B * T, HV, V), np.float64)
    final = np.zeros((N, HV, K, V), np.float64)
    for s, (bos, eos) in enumerate(bounds):
        S = np.zeros((HV, K, V)) if initial_state is None else \
            np.array(initial_state[s], np.float64, copy=True)
        for t in range(bos, eos):
            kt = kf[t][hq]                        # [HV, K]
            qt = qf[t][hq]
            S *= np.exp(gf[t])[:, :, None]
            r = vf[t] - np.einsum('jkv,jk->jv', S, kt)
            S += bf[t][:, None, None] * kt[:, :, None] * r[:, None, :]
            o[t] = scale * np.einsum('jkv,jk->jv', S, qt)
        final[s] = S
    return o.reshape(B, T, HV, V), final
