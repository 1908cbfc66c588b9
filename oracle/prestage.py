"""fp64 pre-stage of the KDA forward: the steps that turn raw projections into the q, k, g, beta
the recurrence reads (test infrastructure).

Per token t and head, on the values the GPU reads (bf16 or fp32, upcast exactly):

  q/k L2 norm     x <- x / sqrt(sum_d x_d^2 + 1e-6) over the key dimension, separately for q and
                  k of every token and q/k head ("KDA源码剖析之FlashKDA（上）", part 6, L2
                  normalisation; the C++ reference of "手撕KDA" section 2.1 applies the same
                  epsilon inside the square root)
  beta sigmoid    beta <- 1 / (1 + exp(-beta_raw)) (the FlashKDA page scales the rows of L by
                  the sigmoid of the raw beta, part 10; the "手撕KDA" C++ reference computes
                  it in its pre-stage, section 2.1)
  gate            g from the raw gate input g_raw with per-head parameters A_log and dt_bias:
                    softplus form   g = -exp(A_log) * softplus(g_raw + dt_bias)
                                    ("手撕KDA" section 2.1, its pre-stage)
                    bounded form    g = lb * sigmoid(exp(A_log) * (g_raw + dt_bias)), lb < 0
                                    ("KDA源码剖析之FlashKDA（上）", part 7, gate activation +
                                    cumsum; "手撕KDA" section 5 uses the same bounded gate)
                  The FlashKDA kernel folds log2(e) into its gate scale to use base-2
                  exponentials; here g stays a natural-log decay, as the recurrence reads it.

Reading (the pages have one head per gate parameter and HV == H): A_log has one entry and
dt_bias one row of K entries per VALUE head, because g and beta are per value head.

``prestage_backward`` is the reverse mode of these steps (the backward of the pre-stage that
the C++ reference of "手撕KDA" section 2.1 runs after its chunk backward), written from the
derivatives of the definitions above:
  l2 norm     y = x r, r = (|x|^2 + eps)^(-1/2):   dx = r dy - r^3 x (x . dy)
  sigmoid     d sigma / dx = sigma (1 - sigma)
  softplus    d softplus / dx = sigma(x)
  gates       softplus form  dg/dx = -exp(A_log) sigma(x),          dg/dA_log = g
              bounded form   dg/dx = lb sigma (1 - sigma) exp(A_log), dg/dA_log = x dg/dx
              (sigma taken at exp(A_log) x); dt_bias and A_log collect their gradients over
              every token.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def l2_normalize(x, eps=L2_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis, in fp64."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)), in fp64 without overflow for large |x|."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + exp(x)), in fp64 without overflow for large x."""
    return np.logaddexp(0.0, np.asarray(x, np.float64))


def gate_activation(g_raw, A_log, dt_bias, mode, lower_bound=-5.0):
    """Per-key-dimension log decay from the raw gate input.

    g_raw [..., HV, K]; A_log [HV]; dt_bias [HV, K] or None (zeros). mode "softplus" or
    "bounded" (lower_bound < 0 for the latter).
    """
    g_raw = np.asarray(g_raw, np.float64)
    HV, K = g_raw.shape[-2], g_raw.shape[-1]
    a = np.exp(np.asarray(A_log, np.float64)).reshape(HV, 1)
    x = g_raw + (0.0 if dt_bias is None else np.asarray(dt_bias, np.float64).reshape(HV, K))
    if mode == "softplus":
        return -a * softplus(x)
    if mode == "bounded":
        return float(lower_bound) * sigmoid(a * x)
    raise ValueError(f"unknown gate mode {mode!r}")


def prestage(q, k, g, beta, qk_l2norm=False, beta_sigmoid=False, gate=None, A_log=None,
             dt_bias=None, lower_bound=-5.0):
    """Apply the selected pre-stage steps; returns fp64 (q, k, g, beta) for the recurrence.

    q, k [B,T,H,K]; g [B,T,HV,K]; beta [B,T,HV]; gate None (g used as given), "softplus" or
    "bounded".
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    if beta_sigmoid:
        beta = sigmoid(beta)
    if gate is not None:
        g = gate_activation(g, A_log, dt_bias, gate, lower_bound)
    return q, k, g, beta


def l2_normalize_vjp(x, dy, eps=L2_EPS):
    """Gradient with respect to x of sum(dy * l2_normalize(x)), over the last axis."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    return r * dy - r ** 3 * x * np.sum(x * dy, axis=-1, keepdims=True)


def gate_activation_vjp(g_raw, A_log, dt_bias, mode, dg, lower_bound=-5.0):
    """Gradients of sum(dg * gate_activation(...)) with respect to g_raw [.., HV, K], A_log
    [HV] and dt_bias [HV, K] (returned even when dt_bias is None: the gradient of a zero
    bias)."""
    g_raw = np.asarray(g_raw, np.float64)
    dg = np.asarray(dg, np.float64)
    HV, K = g_raw.shape[-2], g_raw.shape[-1]
    a = np.exp(np.asarray(A_log, np.float64)).reshape(HV, 1)
    x = g_raw + (0.0 if dt_bias is None else np.asarray(dt_bias, np.float64).reshape(HV, K))
    if mode == "softplus":
        dgdx = -a * sigmoid(x)
        dgda = -a * softplus(x)                       # = g
    elif mode == "bounded":
        s = sigmoid(a * x)
        dgdx = float(lower_bound) * s * (1.0 - s) * a
        dgda = dgdx * x
    else:
        raise ValueError(f"unknown gate mode {mode!r}")
    dx = dg * dgdx
    lead = tuple(range(dx.ndim - 2))
    return dx, np.sum(dg * dgda, axis=lead + (dx.ndim - 1,)), np.sum(dx, axis=lead)


def prestage_backward(q, k, g, beta, dq, dk, dg, dbeta, qk_l2norm=False, beta_sigmoid=False,
                      gate=None, A_log=None, dt_bias=None, lower_bound=-5.0):
    """Gradients with respect to the raw inputs of ``prestage`` given the gradients (dq, dk,
    dg, dbeta) of its outputs. Returns (dq_raw, dk_raw, dg_raw, dbeta_raw, dA_log, ddt_bias);
    the last two are None without a gate."""
    dq = np.asarray(dq, np.float64)
    dk = np.asarray(dk, np.float64)
    dg = np.asarray(dg, np.float64)
    dbeta = np.asarray(dbeta, np.float64)
    if qk_l2norm:
        dq, dk = l2_normalize_vjp(q, dq), l2_normalize_vjp(k, dk)
    if beta_sigmoid:
        s = sigmoid(beta)
        dbeta = dbeta * s * (1.0 - s)
    dA = ddt = None
    if gate is not None:
        dg, dA, ddt = gate_activation_vjp(g, A_log, dt_bias, gate, dg, lower_bound)
    return dq, dk, dg, dbeta, dA, ddt
