"""fp64 gradients of the KDA forward (test infrastructure).

The forward is the token recurrence of recurrent.py: per token t of a sequence, for value head
j and q/k head h,

    S' = diag(exp g_t) S_{t-1};  r = v_t - S'^T k_t;  S_t = S' + beta_t k_t r^T;
    o_t = scale S_t^T q_t

with final_state = S_T. Given the loss gradients do (for o) and dht (for the final state),
``kda_backward_recurrent`` runs the recurrence's reverse mode token by token, newest first,
carrying dS = d loss / d S_t:

    dS  += scale q_t do_t^T                     (o_t reads S_t)
    dq_t = scale S_t do_t
    dr   = beta_t dS^T k_t                      (S_t = S' + beta k r^T)
    dbeta_t = r . (dS^T k_t)
    dk_t = beta_t dS r - S' dr                  (r = v - S'^T k adds -S' dr)
    dv_t = dr
    dS'  = dS - k_t dr^T
    dg_t = rowsum(dS' * S')                     (S' = diag(e^g) S_{t-1}: d/dg_i = S'_i.)
    dS   = diag(exp g_t) dS'                    (now d loss / d S_{t-1})

and dh0 = dS after the first token. dq and dk of a q/k head sum over the value heads of its
group. The derivation is the chain rule applied to the four lines above, in reverse order;
"手撕KDA" section 2.1 (the C++ chunk backward) sweeps the chunks in the same reverse order,
carrying dS from the final-state gradient backwards.

``kda_backward_autograd`` computes the same gradients by PyTorch's reverse-mode
differentiation of the forward written with plain fp64 CPU tensor ops, as an independent check.

``kda_backward_raw`` is the backward of the forward with its pre-stage: the pre-stage
(prestage.py) turns raw inputs into q, k, g, beta, the recurrence's backward gives their
gradients, and the pre-stage's reverse mode carries them back to the raw inputs and to the
gate parameters A_log and dt_bias.
"""
from __future__ import annotations

import numpy as np

from oracle import prestage as PS
from oracle.recurrent import _bounds


def kda_backward_recurrent(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                           do=None, dht=None):
    """Gradients (dq, dk, dv, dg, dbeta, dh0), fp64, shapes like the inputs (dh0 [N,HV,K,V]).

    q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV]; do [B,T,HV,V] or None (zero);
    dht [N,HV,K,V] or None (zero).
    """
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
    N = len(bounds)
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV, K), beta.reshape(B * T, HV)
    dof = (np.zeros((B * T, HV, V)) if do is None
           else np.asarray(do, np.float64).reshape(B * T, HV, V))
    dq = np.zeros((B * T, H, K))
    dk = np.zeros((B * T, H, K))
    dv = np.zeros((B * T, HV, V))
    dg = np.zeros((B * T, HV, K))
    db = np.zeros((B * T, HV))
    dh0 = np.zeros((N, HV, K, V))
    for s, (bos, eos) in enumerate(bounds):
        for j in range(HV):
            h = j // G
            S = (np.zeros((K, V)) if initial_state is None
                 else np.asarray(initial_state, np.float64)[s, j].copy())
            # forward, keeping S' and S of every token
            Sp, St, rr = [], [], []
            for t in range(bos, eos):
                sp = np.exp(gf[t, j])[:, None] * S
                r = vf[t, j] - sp.T @ kf[t, h]
                S = sp + bf[t, j] * np.outer(kf[t, h], r)
                Sp.append(sp)
                St.append(S)
                rr.append(r)
            dS = np.zeros((K, V)) if dht is None else np.asarray(dht, np.float64)[s, j].copy()
            for t in range(eos - 1, bos - 1, -1):
                i = t - bos
                sp, st, r = Sp[i], St[i], rr[i]
                dS += scale * np.outer(qf[t, h], dof[t, j])
                dq[t, h] += scale * st @ dof[t, j]
                dSk = dS.T @ kf[t, h]
                dr = bf[t, j] * dSk
                db[t, j] = r @ dSk
                dk[t, h] += bf[t, j] * (dS @ r) - sp @ dr
                dv[t, j] = dr
                dSp = dS - np.outer(kf[t, h], dr)
                dg[t, j] = np.sum(dSp * sp, axis=1)
                dS = np.exp(gf[t, j])[:, None] * dSp
            dh0[s, j] = dS
    return (dq.reshape(B, T, H, K), dk.reshape(B, T, H, K), dv.reshape(B, T, HV, V),
            dg.reshape(B, T, HV, K), db.reshape(B, T, HV), dh0)


def kda_backward_autograd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                          do=None, dht=None):
    """The same gradients by torch.autograd on the fp64 forward recurrence (CPU)."""
    import torch
    t = lambda x: torch.tensor(np.asarray(x, np.float64), dtype=torch.float64,
                               requires_grad=True)
    q, k, v, g, beta = t(q), t(k), t(v), t(g), t(beta)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    if scale is None:
        scale = K ** -0.5
    bounds = _bounds(B, T, cu_seqlens)
    N = len(bounds)
    h0 = (torch.zeros(N, HV, K, V, dtype=torch.float64) if initial_state is None
          else torch.tensor(np.asarray(initial_state, np.float64)))
    h0.requires_grad_(True)
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV, K), beta.reshape(B * T, HV)
    loss = torch.zeros((), dtype=torch.float64)
    dof = None if do is None else torch.tensor(np.asarray(do, np.float64)).reshape(B * T, HV, V)
    dhf = None if dht is None else torch.tensor(np.asarray(dht, np.float64))
    for s, (bos, eos) in enumerate(bounds):
        for j in range(HV):
            h = j // G
            S = h0[s, j]
            for tt in range(bos, eos):
                sp = torch.exp(gf[tt, j])[:, None] * S
                r = vf[tt, j] - sp.T @ kf[tt, h]
                S = sp + bf[tt, j] * torch.outer(kf[tt, h], r)
                if dof is not None:
                    loss = loss + (scale * S.T @ qf[tt, h]) @ dof[tt, j]
            if dhf is not None:
                loss = loss + (S * dhf[s, j]).sum()
    if not loss.requires_grad:
        z = lambda x: np.zeros(x.shape)
        return z(q), z(k), z(v), z(g), z(beta), np.zeros(h0.shape)
    grads = torch.autograd.grad(loss, [q, k, v, g, beta, h0], allow_unused=True)
    return tuple(np.zeros(x.shape) if gr is None else gr.detach().numpy()
                 for gr, x in zip(grads, [q, k, v, g, beta, h0]))


def kda_backward_raw(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                     do=None, dht=None, qk_l2norm=False, beta_sigmoid=False, gate=None,
                     A_log=None, dt_bias=None, lower_bound=-5.0):
    """Gradients with respect to the RAW inputs of the forward with its pre-stage:
    (dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias); dA_log, ddt_bias are None without a
    gate."""
    qa, ka, ga, ba = PS.prestage(q, k, g, beta, qk_l2norm, beta_sigmoid, gate, A_log, dt_bias,
                                 lower_bound)
    dq, dk, dv, dg, db, dh0 = kda_backward_recurrent(qa, ka, v, ga, ba, scale, initial_state,
                                                     cu_seqlens, do, dht)
    dq, dk, dg, db, dA, ddt = PS.prestage_backward(q, k, g, beta, dq, dk, dg, db, qk_l2norm,
                                                   beta_sigmoid, gate, A_log, dt_bias,
                                                   lower_bound)
    return dq, dk, dv, dg, db, dh0, dA, ddt
