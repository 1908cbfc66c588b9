"""Pins of the oracle's pre-stage reverse mode (oracle/prestage.py: l2_normalize_vjp,
gate_activation_vjp, prestage_backward; oracle/backward.py: kda_backward_raw), CPU only.

  finite diff   <grad, d> == central difference along random directions d of
                L = sum(cotangent * f(x)) for each pre-stage step, and of the full loss
                sum(o * do) + sum(final * dht) through prestage + the fp64 recurrence for every
                raw input and both gate parameters
  autograd      == torch.autograd on the pre-stage written independently here in torch ops
  closed forms  sigmoid'(0) = 1/4; softplus gate with A_log = 0 at x = 0 has slope -1/2 and
                dA_log = g; l2 norm: x . dx = eps r^3 (x . dy), the gradient is (up to eps)
                orthogonal to x
Planted mistakes (each a plausible slip in one VJP) must each fail one of these pins.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import backward as BW
from oracle import prestage as P
from oracle.recurrent import kda_recurrent

RNG = np.random.default_rng(1234)
EPS_FD = 1e-6


def fd_check(f, x, dy, grad, tol=1e-7):
    """<grad, d> against the central difference of sum(dy * f(x + t d)) at t = 0."""
    d = RNG.standard_normal(np.shape(x))
    h = EPS_FD * max(float(np.sqrt(np.mean(np.square(x)))), 1e-3)   # step scaled to x
    fd = (np.sum(dy * f(x + h * d)) - np.sum(dy * f(x - h * d))) / (2 * h)
    an = float(np.sum(grad * d))
    assert abs(fd - an) <= tol * max(1.0, abs(fd)), f"fd {fd:.10g} vs analytic {an:.10g}"


# --------------------------------------------------------------------------- pins as functions

def pin_l2_vjp(vjp):
    for scale in (1e-3, 1.0, 20.0):
        x = RNG.standard_normal((3, 2, 6)) * scale
        dy = RNG.standard_normal(x.shape)
        gx = vjp(x, dy)
        fd_check(P.l2_normalize, x, dy, gx, tol=1e-6)
        r = 1.0 / np.sqrt(np.sum(x * x, -1) + 1e-6)
        assert np.allclose(np.sum(x * gx, -1), 1e-6 * r ** 3 * np.sum(x * dy, -1),
                           rtol=1e-8, atol=1e-12)


def pin_gate_vjp(vjp):
    HV, K = 3, 4
    g_raw = RNG.standard_normal((5, HV, K)) * 2
    A_log = RNG.standard_normal(HV) * 0.5
    dt = RNG.standard_normal((HV, K)) * 0.5
    dg = RNG.standard_normal(g_raw.shape)
    for mode in ("softplus", "bounded"):
        dx, dA, ddt = vjp(g_raw, A_log, dt, mode, dg, -4.0)
        fd_check(lambda z: P.gate_activation(z, A_log, dt, mode, -4.0), g_raw, dg, dx)
        fd_check(lambda a: P.gate_activation(g_raw, a, dt, mode, -4.0), A_log, dg, dA)
        fd_check(lambda b: P.gate_activation(g_raw, A_log, b, mode, -4.0), dt, dg, ddt)
    # closed forms: softplus gate, A_log = 0, x = 0: slope -sigmoid(0) = -1/2, dA_log = g
    z = np.zeros((1, 1, 2))
    dx, dA, ddt = vjp(z, np.zeros(1), None, "softplus", np.ones_like(z))
    assert np.allclose(dx, -0.5, rtol=1e-14)
    assert np.allclose(dA, 2 * -math.log(2.0), rtol=1e-14)
    assert np.allclose(ddt, -0.5, rtol=1e-14)


def pin_prestage_backward(bwd):
    B, T, H, HV, K = 1, 6, 2, 4, 5
    q = RNG.standard_normal((B, T, H, K))
    k = RNG.standard_normal((B, T, H, K))
    g = RNG.standard_normal((B, T, HV, K))
    b = RNG.standard_normal((B, T, HV))
    A_log = RNG.standard_normal(HV) * 0.5
    dt = RNG.standard_normal((HV, K)) * 0.5
    cot = [RNG.standard_normal(x.shape) for x in (q, k, g, b)]
    for mode in ("softplus", "bounded"):
        got = bwd(q, k, g, b, *cot, True, True, mode, A_log, dt, -3.0)
        # torch autograd on the definitions, written independently in torch ops
        tt = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
        tq, tk, tg, tb, ta, td = map(tt, (q, k, g, b, A_log, dt))
        nq = tq / torch.sqrt((tq * tq).sum(-1, keepdim=True) + 1e-6)
        nk = tk / torch.sqrt((tk * tk).sum(-1, keepdim=True) + 1e-6)
        sb = torch.sigmoid(tb)
        xg = tg + td
        ea = torch.exp(ta)[:, None]
        ag = (-ea * torch.nn.functional.softplus(xg) if mode == "softplus"
              else -3.0 * torch.sigmoid(ea * xg))
        L = sum((y * torch.tensor(c)).sum() for y, c in zip((nq, nk, ag, sb), cot))
        ref = torch.autograd.grad(L, [tq, tk, tg, tb, ta, td])
        for name, a, r in zip(("q", "k", "g", "beta", "A_log", "dt_bias"), got, ref):
            assert np.allclose(a, r.numpy(), rtol=1e-11, atol=1e-13), (mode, name)
    # beta sigmoid closed form: sigmoid'(0) = 1/4
    z = np.zeros((1, 2, HV))
    out = bwd(q[:, :2], k[:, :2], g[:, :2], z, q[:, :2], k[:, :2], g[:, :2], np.ones_like(z),
              False, True, None)
    assert np.allclose(out[3], 0.25, rtol=1e-15)
    assert out[4] is None and out[5] is None


def pin_raw_backward(bwd):
    """Full loss through prestage + recurrence, central differences for every raw input."""
    B, T, H, HV, K, V = 1, 7, 1, 2, 4, 3
    q = RNG.standard_normal((B, T, H, K))
    k = RNG.standard_normal((B, T, H, K))
    v = RNG.standard_normal((B, T, HV, V))
    g = RNG.standard_normal((B, T, HV, K))
    b = RNG.standard_normal((B, T, HV))
    A_log = RNG.standard_normal(HV) * 0.3
    dt = RNG.standard_normal((HV, K)) * 0.3
    S0 = RNG.standard_normal((1, HV, K, V)) * 0.3
    do = RNG.standard_normal((B, T, HV, V))
    dht = RNG.standard_normal((1, HV, K, V))
    for mode in ("softplus", "bounded"):
        args = [q, k, v, g, b, S0, A_log, dt]

        def L(a):
            qa, ka, ga, ba = P.prestage(a[0], a[1], a[3], a[4], True, True, mode, a[6], a[7],
                                        -4.0)
            o, fin = kda_recurrent(qa, ka, a[2], ga, ba, 0.6, a[5])
            return float(np.sum(o * do) + np.sum(fin * dht))

        got = bwd(q, k, v, g, b, 0.6, S0, None, do, dht, True, True, mode, A_log, dt, -4.0)
        order = [0, 1, 2, 3, 4, 5, 6, 7]     # q, k, v, g, beta, h0, A_log, dt_bias
        for idx, gr in zip(order, got):
            d = RNG.standard_normal(np.shape(args[idx]))
            ap, am = list(args), list(args)
            ap[idx] = args[idx] + EPS_FD * d
            am[idx] = args[idx] - EPS_FD * d
            fd = (L(ap) - L(am)) / (2 * EPS_FD)
            an = float(np.sum(gr * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (mode, idx, fd, an)


# --------------------------------------------------------------------------- the oracle passes

def test_l2_vjp_pins():
    pin_l2_vjp(P.l2_normalize_vjp)


def test_gate_vjp_pins():
    pin_gate_vjp(P.gate_activation_vjp)


def test_prestage_backward_pins():
    pin_prestage_backward(P.prestage_backward)


def test_raw_backward_matches_finite_differences():
    pin_raw_backward(BW.kda_backward_raw)


# --------------------------------------------------------------------------- planted mistakes

def _l2_vjp_no_projection(x, dy, eps=1e-6):
    x = np.asarray(x, np.float64)
    return dy / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _gate_vjp_no_exp(g_raw, A_log, dt_bias, mode, dg, lower_bound=-5.0):
    dx, dA, ddt = P.gate_activation_vjp(g_raw, A_log, dt_bias, mode, dg, lower_bound)
    a = np.exp(np.asarray(A_log, np.float64)).reshape(-1, 1)
    return dx / a, dA, ddt / a                      # slope without its exp(A_log) factor


def _gate_vjp_dA_without_x(g_raw, A_log, dt_bias, mode, dg, lower_bound=-5.0):
    dx, dA, ddt = P.gate_activation_vjp(g_raw, A_log, dt_bias, mode, dg, lower_bound)
    return dx, np.sum(dx, axis=tuple(range(dx.ndim - 2)) + (dx.ndim - 1,)), ddt


def _prestage_bwd_sigmoid_slope(q, k, g, beta, dq, dk, dg, dbeta, qk_l2norm=False,
                                beta_sigmoid=False, gate=None, A_log=None, dt_bias=None,
                                lower_bound=-5.0):
    out = list(P.prestage_backward(q, k, g, beta, dq, dk, dg, dbeta, qk_l2norm, False, gate,
                                   A_log, dt_bias, lower_bound))
    if beta_sigmoid:
        out[3] = np.asarray(dbeta) * P.sigmoid(beta)  # sigma instead of sigma (1 - sigma)
    return tuple(out)


def _prestage_bwd_same_norm(q, k, g, beta, dq, dk, dg, dbeta, qk_l2norm=False,
                            beta_sigmoid=False, gate=None, A_log=None, dt_bias=None,
                            lower_bound=-5.0):
    out = list(P.prestage_backward(q, k, g, beta, dq, dk, dg, dbeta, qk_l2norm, beta_sigmoid,
                                   gate, A_log, dt_bias, lower_bound))
    if qk_l2norm:
        out[1] = P.l2_normalize_vjp(q, dk)          # k's gradient through q's norm
    return tuple(out)


MUTANTS = [
    ("l2 vjp without the projection", pin_l2_vjp, _l2_vjp_no_projection),
    ("gate slope without exp(A_log)", pin_gate_vjp, _gate_vjp_no_exp),
    ("bounded dA_log without x", pin_gate_vjp, _gate_vjp_dA_without_x),
    ("beta sigmoid slope sigma", pin_prestage_backward, _prestage_bwd_sigmoid_slope),
    ("k through q's norm", pin_prestage_backward, _prestage_bwd_same_norm),
]


@pytest.mark.parametrize("name,pin,impl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_prestage_backward_mistakes_are_caught(name, pin, impl):
    with pytest.raises(AssertionError):
        pin(impl)
