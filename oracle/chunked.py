"""fp64 chunked (WY / UT) form of the KDA forward, as the pages lay it out (test infrastructure).

Source: "手撕KDA" ("KDA by hand"), section 1 (the naive_chunk_kda routine), with the tail
handling of "KDA源码剖析之FlashKDA（上）" (part 7: rows past the end of a sequence get k = 0,
g = 0) so that any length is accepted.

Per sequence, per value head j (q/k head h = j // G), per chunk of C tokens with in-chunk index
i = 0..C-1:

  Gam_i   = sum_{tau <= i} g_tau                    inclusive in-chunk cumsum, per key dim
  gam     = Gam_{C-1}                               total chunk decay (log)
  L_ij    = beta_i sum_d k_id k_jd exp(Gam_id - Gam_jd)            i > j, else 0
  A       = (I + L)^{-1} diag(beta)
  w       = A (exp(Gam) * k)           u = A v
  qd      = scale * q * exp(Gam)       kr = k * exp(gam - Gam)
  Mqk_ij  = scale sum_d q_id k_jd exp(Gam_id - Gam_jd)             i >= j, else 0
  then, over chunks in order, with S the state at the chunk start:
  delta   = u - w S
  o       = qd S + Mqk delta
  S      <- diag(exp(gam)) S + kr^T delta

The oracle evaluates the decayed Gram matrices with the exponent of the *difference* (never the
factorised exp(Gam) * exp(-Gam)), and the inverse by row-wise forward substitution as the
listing does. Mathematically the result equals the token recurrence for every chunk size C
(the chunk-size independence the pages rely on in section 5 of "手撕KDA").
"""
from __future__ import annotations

import numpy as np

from .recurrent import _bounds


def inverse_forward_substitution(L):
    """(I + L)^{-1} for strictly lower-triangular L (..., n, n), row by row.

    Row i of X = (I + L)^{-1} satisfies X_i = e_i - sum_{j < i} L_ij X_j, the sequential solve
    of the naive listing ("手撕KDA", section 1)."""
    L = np.asarray(L, np.float64)
    n = L.shape[-1]
    X = np.zeros_like(L)
    for i in range(n):
        X[..., i, i] = 1.0
        for j in range(i):
            X[..., i, :] -= L[..., i, j, None] * X[..., j, :]
    return X


def inverse_neumann(L):
    """(I + L)^{-1} = (I - L)(I + L^2)(I + L^4)(I + L^8) ... for strictly lower-triangular L.

    Exact because L is nilpotent (L^n = 0 for n x n): the product expands to
    sum_{m=0}^{n-1} (-L)^m. Source: "KDA源码剖析之FlashKDA（上）", part 12 (Neumann series
    inverse by repeated squaring), and the FlashKDA 16x16 Neumann-inverse walkthrough page."""
    L = np.asarray(L, np.float64)
    n = L.shape[-1]
    eye = np.broadcast_to(np.eye(n), L.shape)
    inv = eye - L
    P = L
    span = 2                     # inv currently equals sum_{m < span} (-L)^m
    while span < n:
        P = P @ P                # L^(span)
        inv = inv + inv @ P
        span *= 2
    return inv


def chunk_prepare(q, k, v, g, beta, scale, C):
    """Per-chunk intermediates for one sequence and one value head.

    q, k [L, K] (the value head's q/k rows), v [L, V], g [L, K], beta [L]. The sequence is
    padded to a multiple of C with k = q = v = 0, g = 0, beta = 0 rows. Returns a dict of
    arrays with a leading chunk axis: Gam [NC,C,K], gam [NC,K], L [NC,C,C], A [NC,C,C],
    w [NC,C,K], u [NC,C,V], qd [NC,C,K], kr [NC,C,K], Mqk [NC,C,C], eg [NC,K]; n_valid [NC].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    Ls, K = k.shape
    V = v.shape[1]
    NC = -(-Ls // C)
    pad = NC * C - Ls

    def padrows(x):
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:])], 0) if pad else x

    q, k, v, g, beta = [padrows(x).reshape((NC, C) + x.shape[1:]) for x in (q, k, v, g, beta)]
    Gam = np.cumsum(g, axis=1)                            # [NC, C, K]
    gam = Gam[:, -1, :]                                   # [NC, K]
    ii, jj = np.meshgrid(np.arange(C), np.arange(C), indexing='ij')
    strict = ii > jj
    incl = ii >= jj
    diff = Gam[:, :, None, :] - Gam[:, None, :, :]        # [NC, C(i), C(j), K]
    # exponent of the difference, evaluated only where it is <= 0 (i >= j)
    dec = np.where(incl[None, :, :, None], np.exp(np.where(incl[None, :, :, None], diff, 0.0)),
                   0.0)
    kk = np.einsum('nid,njd,nijd->nij', k, k, dec)
    Lm = np.where(strict[None], beta[:, :, None] * kk, 0.0)
    Ainv = inverse_forward_substitution(Lm)
    A = Ainv * beta[:, None, :]                           # (I+L)^{-1} diag(beta)
    w = A @ (np.exp(Gam) * k)
    u = A @ v
    qd = scale * q * np.exp(Gam)
    kr = k * np.exp(gam[:, None, :] - Gam)
    Mqk = np.where(incl[None], scale * np.einsum('nid,njd,nijd->nij', q, k, dec), 0.0)
    n_valid = np.minimum(C, Ls - C * np.arange(NC))
    return dict(Gam=Gam, gam=gam, L=Lm, A=A, w=w, u=u, qd=qd, kr=kr, Mqk=Mqk,
                eg=np.exp(gam), n_valid=n_valid)


def chunk_state_pass(prep, S0):
    """Run the chunk-sequential state pass of one sequence/head. Returns (o [L,V], S)."""
    S = np.array(S0, np.float64, copy=True)
    outs = []
    for c in range(prep['w'].shape[0]):
        delta = prep['u'][c] - prep['w'][c] @ S
        outs.append(prep['qd'][c] @ S + prep['Mqk'][c] @ delta)
        S = prep['eg'][c][:, None] * S + prep['kr'][c].T @ delta
    o = np.concatenate(outs, 0)
    return o, S


def kda_chunked(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, C=16):
    """KDA forward by the chunked form with chunk size C, in fp64. Same signature and outputs
    as recurrent.kda_recurrent."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    if scale is None:
        scale = K ** -0.5
    bounds = _bounds(B, T, cu_seqlens)
    qf = q.reshape(B * T, H, K)
    kf = k.reshape(B * T, H, K)
    vf = v.reshape(B * T, HV, V)
    gf = g.reshape(B * T, HV, K)
    bf = beta.reshape(B * T, HV)
    o = np.zeros((B * T, HV, V))
    final = np.zeros((len(bounds), HV, K, V))
    for s, (bos, eos) in enumerate(bounds):
        for j in range(HV):
            h = j // G
            S0 = np.zeros((K, V)) if initial_state is None else initial_state[s][j]
            if eos == bos:
                final[s, j] = S0
                continue
            prep = chunk_prepare(qf[bos:eos, h], kf[bos:eos, h], vf[bos:eos, j],
                                 gf[bos:eos, j], bf[bos:eos, j], scale, C)
            oj, S = chunk_state_pass(prep, S0)
            o[bos:eos, j] = oj[:eos - bos]
            final[s, j] = S
    return o.reshape(B, T, HV, V), final
