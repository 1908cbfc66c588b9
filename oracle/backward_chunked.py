"""fp64 chunked backward of the KDA forward, as the GPU kernels organise it (test infrastructure).

The token recurrence's reverse mode (backward.py) is the definition of the gradients. This module
states the same gradients in the chunked form of "手撕KDA" section 1 (chunks of 16 tokens), the
way the C++ chunk backward of that page's section 2.1 sweeps them: states recorded at every
chunk start by a forward pass, the state gradient Lam = d loss / d S carried newest chunk first,
then every chunk's own quantities back-propagated to its tokens. It is pinned against
backward.py (tests/test_oracle_backward.py) and shares no code with the HIP kernels.

Per chunk, with S the state at its start, Gam the in-chunk cumsum of g, gam = Gam at its last
row, and rows past the sequence end padded with q = k = v = g = beta = 0:
    KD = k e^Gam,  QD = scale q e^Gam,  KR = k e^(gam - Gam),  E = e^gam
    G_ij = sum_d k_id k_jd e^(Gam_id - Gam_jd)  (i > j),  Mqk_ij = scale sum_d q_id k_jd e^(...)
    (i >= j),  L = diag(beta) G,  X = (I + L)^-1,  A = X diag(beta),  W = A KD,  U = A v
    delta = U - W S,  O = QD S + Mqk delta,  S_next = diag(E) S + KR^T delta
Reverse mode of those lines, with Lam the gradient of S_next and dO that of O:
    dDelta = Mqk^T dO + KR Lam;  Lam_prev = diag(E) Lam + QD^T dO - W^T dDelta
    dQD = dO S^T, dKR = delta Lam^T, dW = -dDelta S^T, dE = rowsum(Lam * S),
    dMqk = tril(dO delta^T), dA = dDelta v^T + dW KD^T, dv = A^T dDelta, dKD = A^T dW
    dbeta_j += sum_i dA_ij X_ij;  dX = dA diag(beta);  dL = -strict_tril(X^T dX X^T)
    dbeta_i += sum_j dL_ij G_ij;  dG = diag(beta) dL
and to the tokens, per key dim, every pair i > j of G and Mqk with e = e^(Gam_i - Gam_j):
    dk_i += dG_ij k_j e,  dq_i += dMqk_ij scale k_j e,
    dk_j += (dG_ij k_i + dMqk_ij scale q_i) e,  dGam_i += c k_j,  dGam_j -= c k_j
    (c = (dG_ij k_i + dMqk_ij scale q_i) e), the diagonal of Mqk (no decay), and the per-token
    terms of KD, QD, KR; then dgam = dE E + sum_t dKR_t KR_t and dg_tau = sum_{t >= tau}
    dGam_t + dgam (the reverse cumsum).
"""
from __future__ import annotations

import numpy as np

from oracle.recurrent import _bounds

C = 16


def _chunk_records(q, k, v, g, beta, scale):
    """Per-chunk quantities of one (sequence, value head); inputs padded to a multiple of C."""
    gm = np.cumsum(g, axis=0)
    G = np.zeros((C, C))
    Mq = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            e = np.exp(gm[i] - gm[j])
            if i > j:
                G[i, j] = np.sum(k[i] * k[j] * e)
            Mq[i, j] = scale * np.sum(q[i] * k[j] * e)
    X = np.linalg.inv(np.eye(C) + beta[:, None] * G)
    A = X * beta[None, :]
    KD = k * np.exp(gm)
    return dict(q=q, k=k, v=v, gm=gm, beta=beta, G=G, Mq=Mq, X=X, A=A, KD=KD,
                QD=scale * q * np.exp(gm), KR=k * np.exp(gm[-1] - gm), E=np.exp(gm[-1]),
                W=A @ KD, U=A @ v)


def _chunk_token_grads(r, S, Lam, dO, scale):
    """dq, dk, dv, dg, dbeta of one chunk's tokens from S (its start state), Lam (the state
    gradient at its end) and dO."""
    A, X, G, Mq, KR, W, KD = r["A"], r["X"], r["G"], r["Mq"], r["KR"], r["W"], r["KD"]
    q, k, v, gm, beta = r["q"], r["k"], r["v"], r["gm"], r["beta"]
    delta = r["U"] - W @ S
    dd = Mq.T @ dO + KR @ Lam
    dQD, dKR, dW = dO @ S.T, delta @ Lam.T, -dd @ S.T
    dE = np.sum(Lam * S, axis=1)
    dMq = np.tril(dO @ delta.T)
    dA = dd @ v.T + dW @ KD.T
    dv = A.T @ dd
    dKD = A.T @ dW
    dbeta = np.sum(dA * X, axis=0)
    dX = dA * beta[None, :]
    dL = np.tril(-(X.T @ dX @ X.T), -1)
    dbeta = dbeta + np.sum(dL * G, axis=1)
    dG = beta[:, None] * dL
    et, ert = np.exp(gm), np.exp(gm[-1] - gm)
    dk = dKD * et + dKR * ert
    dq = scale * dQD * et
    dgam_t = (dKD * k + scale * dQD * q) * et - dKR * k * ert
    for i in range(C):
        wd = dMq[i, i] * scale            # diagonal of Mqk: q_i . k_i, no decay
        dq[i] += wd * k[i]
        dk[i] += wd * q[i]
        for j in range(i):
            e = np.exp(gm[i] - gm[j])
            w1, w2 = dG[i, j] * e, dMq[i, j] * scale * e
            dk[i] += w1 * k[j]
            dq[i] += w2 * k[j]
            c = w1 * k[i] + w2 * q[i]
            dk[j] += c
            dgam_t[i] += c * k[j]
            dgam_t[j] -= c * k[j]
    dgam = r["E"] * dE + np.sum(dKR * KR, axis=0)
    dg = np.cumsum(dgam_t[::-1], axis=0)[::-1] + dgam
    return dq, dk, dv, dg, dbeta


def kda_backward_chunked(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                         do=None, dht=None):
    """Gradients (dq, dk, dv, dg, dbeta, dh0) in fp64 by the chunked reverse sweep; arguments and
    shapes as oracle.backward.kda_backward_recurrent."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    Gq = HV // H
    if scale is None:
        scale = K ** -0.5
    bounds = _bounds(B, T, cu_seqlens)
    N = len(bounds)
    flat = lambda x: x.reshape(B * T, *x.shape[2:])
    qf, kf, vf, gf, bf = flat(q), flat(k), flat(v), flat(g), flat(beta)
    dof = np.zeros((B * T, HV, V)) if do is None else flat(np.asarray(do, np.float64))
    out = [np.zeros((B * T, H, K)), np.zeros((B * T, H, K)), np.zeros((B * T, HV, V)),
           np.zeros((B * T, HV, K)), np.zeros((B * T, HV))]
    dh0 = np.zeros((N, HV, K, V))
    for s, (bos, eos) in enumerate(bounds):
        L = eos - bos
        nc = (L + C - 1) // C
        pad = lambda x: np.concatenate([x, np.zeros((nc * C - L,) + x.shape[1:])])
        for j in range(HV):
            h = j // Gq
            recs = [_chunk_records(*(pad(x)[C * c:C * c + C] for x in (
                        qf[bos:eos, h], kf[bos:eos, h], vf[bos:eos, j], gf[bos:eos, j],
                        bf[bos:eos, j])), scale) for c in range(nc)]
            dO = pad(dof[bos:eos, j])
            S = (np.zeros((K, V)) if initial_state is None
                 else np.asarray(initial_state, np.float64)[s, j].copy())
            starts = []
            for r in recs:                                   # states at every chunk start
                starts.append(S)
                S = r["E"][:, None] * S + r["KR"].T @ (r["U"] - r["W"] @ S)
            Lam = np.zeros((K, V)) if dht is None else np.asarray(dht, np.float64)[s, j].copy()
            ends = [None] * nc
            for c in range(nc - 1, -1, -1):                 # state gradient, newest first
                r, dOc = recs[c], dO[C * c:C * c + C]
                ends[c] = Lam
                dd = r["Mq"].T @ dOc + r["KR"] @ Lam
                Lam = r["E"][:, None] * Lam + r["QD"].T @ dOc - r["W"].T @ dd
            dh0[s, j] = Lam
            for c in range(nc):                              # every chunk on its own
                grads = _chunk_token_grads(recs[c], starts[c], ends[c], dO[C * c:C * c + C],
                                           scale)
                n = min(C, L - C * c)
                t0 = bos + C * c
                out[0][t0:t0 + n, h] += grads[0][:n]
                out[1][t0:t0 + n, h] += grads[1][:n]
                out[2][t0:t0 + n, j] = grads[2][:n]
                out[3][t0:t0 + n, j] = grads[3][:n]
                out[4][t0:t0 + n, j] = grads[4][:n]
    shapes = [(B, T, H, K), (B, T, H, K), (B, T, HV, V), (B, T, HV, K), (B, T, HV)]
    return tuple(x.reshape(sh) for x, sh in zip(out, shapes)) + (dh0,)
