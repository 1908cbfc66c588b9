"""Pins of the oracle's pre-stage (oracle/prestage.py) against closed forms, library routines
and an independent scalar implementation (CPU only).

  l2 norm     norm of the result = |x| / sqrt(|x|^2 + eps); direction kept; rows normalised
              independently (scalar loop with math.sqrt); a zero row stays zero
  sigmoid     sigmoid(ln a) = a / (1 + a); sigmoid(x) + sigmoid(-x) = 1; scipy.special.expit;
              finite at |x| = 1000
  softplus    softplus(ln a) = ln(1 + a); softplus(x) - softplus(-x) = x; numpy log1p(exp);
              asymptote x for large x
  gates       softplus form with A_log = 0: exp(g) = 1 / (1 + a) for g_raw = ln a; A_log = ln 2
              doubles g; dt_bias shifts the input; bounded form: lb / 2 at zero input, inside
              (lb, 0) otherwise; parameters indexed by value head
  composed    the recurrence on pre-staged raw inputs == the recurrence on inputs pre-staged
              by hand with the scalar routines
Planted mistakes in copies of the pre-stage must each fail one of these pins.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special

from oracle import prestage as P
from oracle.recurrent import kda_recurrent

RNG = np.random.default_rng(77)


# --------------------------------------------------------------------------- pins as functions

def pin_l2(l2):
    x = RNG.standard_normal((3, 5, 2, 7))
    for s in (1e-4, 1.0, 30.0):                       # eps matters at the small scale
        y = l2(s * x)
        n = np.sqrt(np.sum((s * x) ** 2, axis=-1))
        assert np.allclose(np.linalg.norm(y, axis=-1), n / np.sqrt(n * n + 1e-6), rtol=1e-12)
        cos = np.sum(y * x, axis=-1) / (np.linalg.norm(y, axis=-1) * np.linalg.norm(x, axis=-1))
        assert np.allclose(cos, 1.0, atol=1e-12)
    y = l2(x)
    for idx in np.ndindex(x.shape[:-1]):              # independent scalar implementation
        row = [float(v) for v in x[idx]]
        r = 1.0 / math.sqrt(sum(v * v for v in row) + 1e-6)
        assert np.allclose(y[idx], [v * r for v in row], rtol=1e-13)
    assert np.all(l2(np.zeros((2, 4))) == 0)


def pin_sigmoid(sig):
    a = np.array([0.25, 1.0, 3.0, 10.0])
    assert np.allclose(sig(np.log(a)), a / (1 + a), rtol=1e-14)
    x = RNG.standard_normal(50) * 6
    assert np.allclose(sig(x) + sig(-x), 1.0, atol=1e-15)
    assert np.allclose(sig(x), scipy.special.expit(x), rtol=1e-14)
    big = sig(np.array([-1000.0, 1000.0]))
    assert np.all(np.isfinite(big)) and big[0] == 0.0 and big[1] == 1.0


def pin_softplus(sp):
    a = np.array([0.1, 1.0, 2.0, 7.0])
    assert np.allclose(sp(np.log(a)), np.log1p(a), rtol=1e-14)
    x = RNG.standard_normal(50) * 5
    assert np.allclose(sp(x) - sp(-x), x, atol=1e-13)
    assert np.allclose(sp(x), np.log1p(np.exp(x)), rtol=1e-13)
    assert abs(sp(np.array([800.0]))[0] - 800.0) < 1e-12


def pin_gates(gate):
    HV, K = 3, 4
    a = np.array([0.5, 1.0, 4.0, 9.0])
    g_raw = np.broadcast_to(np.log(a), (2, HV, K)).copy()
    g = gate(g_raw, np.zeros(HV), None, "softplus")
    assert np.allclose(np.exp(g), 1.0 / (1.0 + a), rtol=1e-13)
    A_log = np.array([0.0, math.log(2.0), 0.0])       # head 1 doubles, heads 0 and 2 do not
    g2 = gate(g_raw, A_log, None, "softplus")
    assert np.allclose(g2[:, 1], 2 * g[:, 1], rtol=1e-13)
    assert np.allclose(g2[:, [0, 2]], g[:, [0, 2]], rtol=1e-13)
    dt = RNG.standard_normal((HV, K))
    g3 = gate(-dt[None] + np.zeros((2, HV, K)), np.zeros(HV), dt, "softplus")
    assert np.allclose(g3, -math.log(2.0), rtol=1e-13)  # softplus(0) = ln 2
    lb = -5.0
    g4 = gate(-dt[None] + np.zeros((2, HV, K)), RNG.standard_normal(HV), dt, "bounded", lb)
    assert np.allclose(g4, lb / 2, rtol=1e-13)          # sigmoid(0) = 1/2
    x = RNG.standard_normal((6, HV, K)) * 3
    g5 = gate(x, RNG.standard_normal(HV), dt, "bounded", lb)
    assert np.all(g5 < 0) and np.all(g5 > lb)
    # bounded form against sigmoid(ln a) = a / (1 + a): exp(A_log) * x = ln a
    A1 = np.full(HV, math.log(2.0))
    g6 = gate(np.broadcast_to(np.log(a) / 2, (1, HV, K)).copy(), A1, None, "bounded", lb)
    assert np.allclose(g6, lb * a / (1 + a), rtol=1e-13)


# --------------------------------------------------------------------------- the oracle passes

def test_l2_norm_pins():
    pin_l2(P.l2_normalize)


def test_sigmoid_pins():
    pin_sigmoid(P.sigmoid)


def test_softplus_pins():
    pin_softplus(P.softplus)


def test_gate_pins():
    pin_gates(P.gate_activation)


def test_prestage_composed_with_the_recurrence():
    B, T, H, HV, K, V = 1, 9, 1, 2, 5, 3
    q = RNG.standard_normal((B, T, H, K))
    k = RNG.standard_normal((B, T, H, K))
    v = RNG.standard_normal((B, T, HV, V))
    g_raw = RNG.standard_normal((B, T, HV, K))
    b_raw = RNG.standard_normal((B, T, HV))
    A_log = RNG.standard_normal(HV) * 0.5
    dt = RNG.standard_normal((HV, K)) * 0.5
    for mode in ("softplus", "bounded"):
        qn, kn, g, beta = P.prestage(q, k, g_raw, b_raw, True, True, mode, A_log, dt, -4.0)
        # by hand, scalar routines only
        qh = np.empty_like(q); kh = np.empty_like(k); gh = np.empty_like(g_raw)
        bh = np.empty_like(b_raw)
        for t in range(T):
            for h in range(H):
                for src, dst in ((q, qh), (k, kh)):
                    r = 1 / math.sqrt(sum(float(x) ** 2 for x in src[0, t, h]) + 1e-6)
                    dst[0, t, h] = src[0, t, h] * r
            for j in range(HV):
                bh[0, t, j] = 1 / (1 + math.exp(-b_raw[0, t, j]))
                for d in range(K):
                    x = g_raw[0, t, j, d] + dt[j, d]
                    if mode == "softplus":
                        gh[0, t, j, d] = -math.exp(A_log[j]) * math.log1p(math.exp(x))
                    else:
                        gh[0, t, j, d] = -4.0 / (1 + math.exp(-math.exp(A_log[j]) * x))
        o1, f1 = kda_recurrent(qn, kn, v, g, beta, 0.4)
        o2, f2 = kda_recurrent(qh, kh, v, gh, bh, 0.4)
        assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14)
        assert np.allclose(f1, f2, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- planted mistakes

def _l2_no_eps(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _l2_eps_outside(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)


def _l2_wrong_axis(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-2, keepdims=True) + eps)


def _sig_wrong_sign(x):
    return 1.0 / (1.0 + np.exp(np.asarray(x, np.float64)))


def _softplus_plain_exp(x):
    return np.exp(np.asarray(x, np.float64))


def _gate_no_alog(g_raw, A_log, dt_bias, mode, lower_bound=-5.0):
    return P.gate_activation(g_raw, np.zeros_like(np.asarray(A_log, np.float64)), dt_bias, mode,
                             lower_bound)


def _gate_linear_alog(g_raw, A_log, dt_bias, mode, lower_bound=-5.0):
    # A_log used as a plain factor instead of exp(A_log)
    g_raw = np.asarray(g_raw, np.float64)
    HV, K = g_raw.shape[-2], g_raw.shape[-1]
    a = np.asarray(A_log, np.float64).reshape(HV, 1)
    x = g_raw + (0.0 if dt_bias is None else np.asarray(dt_bias, np.float64).reshape(HV, K))
    if mode == "softplus":
        return -a * P.softplus(x)
    return float(lower_bound) * P.sigmoid(a * x)


def _gate_bias_per_qk_head(g_raw, A_log, dt_bias, mode, lower_bound=-5.0):
    # dt_bias rows taken from head 0 for every value head
    d = None if dt_bias is None else np.broadcast_to(np.asarray(dt_bias)[:1], np.shape(dt_bias))
    return P.gate_activation(g_raw, A_log, d, mode, lower_bound)


MUTANTS = [
    ("l2 without eps", pin_l2, _l2_no_eps),
    ("l2 eps outside the root", pin_l2, _l2_eps_outside),
    ("l2 over the wrong axis", pin_l2, _l2_wrong_axis),
    ("sigmoid of -x", pin_sigmoid, _sig_wrong_sign),
    ("softplus as exp", pin_softplus, _softplus_plain_exp),
    ("gate without A_log", pin_gates, _gate_no_alog),
    ("gate with A_log as a factor", pin_gates, _gate_linear_alog),
    ("gate bias of one head for all", pin_gates, _gate_bias_per_qk_head),
]


@pytest.mark.parametrize("name,pin,impl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_prestage_mistakes_are_caught(name, pin, impl):
    with pytest.raises(AssertionError):
        pin(impl)
