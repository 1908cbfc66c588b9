"""Pins of the oracle's backward (oracle/backward.py) against things other than itself (CPU).

  autograd     the hand-derived reverse recurrence == torch.autograd on the fp64 forward
  finite diff  <grad, d> == central difference of L = sum(o * do) + sum(final * dht) along
               random directions d, for every input (q, k, v, g, beta, h0), through the fp64
               forward recurrence (oracle/recurrent.py)
  zero loss    do = 0, dht = 0 gives zero gradients
  decay only   beta = 0: dh0 = exp(sum of g) * dht elementwise (final = exp(sum g) h0)
Planted mistakes (copies of the reverse recurrence with one line changed) must each fail the
finite-difference pin.

The C backward (oracle/kda_oracle_bwd.c, the fast oracle of the full-size GPU tests) is pinned
the same way: central differences of the fp64 forward, including sequences that span several
of its 256-token checkpoint segments; the decay-only and zero-loss cases; and agreement with
the Python reverse recurrence to 1e-12 on fp32-valued inputs.
"""
from __future__ import annotations

import inspect
import math

import numpy as np
import pytest

from oracle import backward as BW
from oracle.recurrent import kda_recurrent

RNG = np.random.default_rng(99)


def rand_case(B=1, T=9, H=1, HV=2, K=4, V=3, cu=None, h0=True):
    Bt = B if cu is None else 1
    Tt = T if cu is None else int(cu[-1])
    N = Bt if cu is None else len(cu) - 1
    q = RNG.standard_normal((Bt, Tt, H, K)) * 0.5
    k = RNG.standard_normal((Bt, Tt, H, K)) * 0.5
    v = RNG.standard_normal((Bt, Tt, HV, V))
    g = -RNG.uniform(0.01, 0.5, (Bt, Tt, HV, K))
    beta = RNG.uniform(0.1, 0.9, (Bt, Tt, HV))
    S0 = RNG.standard_normal((N, HV, K, V)) * 0.3 if h0 else None
    do = RNG.standard_normal((Bt, Tt, HV, V))
    dht = RNG.standard_normal((N, HV, K, V))
    return q, k, v, g, beta, 0.7, S0, cu, do, dht


def loss(q, k, v, g, beta, scale, S0, cu, do, dht):
    o, fin = kda_recurrent(q, k, v, g, beta, scale, S0, cu)
    return float(np.sum(o * do) + np.sum(fin * dht))


def pin_finite_differences(bwd, case):
    q, k, v, g, beta, scale, S0, cu, do, dht = case
    grads = bwd(q, k, v, g, beta, scale, S0, cu, do, dht)
    names = ["q", "k", "v", "g", "beta", "h0"]
    args = [q, k, v, g, beta, S0]
    eps = 1e-6
    for idx, (name, x, gr) in enumerate(zip(names, args, grads)):
        if x is None:
            continue
        d = RNG.standard_normal(x.shape)
        def L(xx):
            a = list(args)
            a[idx] = xx
            return loss(*a[:5], scale, a[5], cu, do, dht)
        fd = (L(x + eps * d) - L(x - eps * d)) / (2 * eps)
        an = float(np.sum(gr * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"d{name}: fd {fd:.9g} vs {an:.9g}"


CASES = {
    "dense_gva": dict(B=2, T=7, H=1, HV=2, K=4, V=3),
    "varlen_empty": dict(H=2, HV=2, K=3, V=2, cu=np.array([0, 5, 5, 11])),
    "one_token": dict(B=1, T=1, H=1, HV=1, K=3, V=2),
    "no_h0": dict(B=1, T=6, H=1, HV=1, K=5, V=4, h0=False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_finite_differences(name):
    pin_finite_differences(BW.kda_backward_recurrent, rand_case(**CASES[name]))


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_autograd(name):
    case = rand_case(**CASES[name])
    a = BW.kda_backward_recurrent(*case)
    b = BW.kda_backward_autograd(*case)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-11, atol=1e-12)


def test_zero_loss_gradient_is_zero():
    q, k, v, g, beta, scale, S0, cu, do, dht = rand_case()
    grads = BW.kda_backward_recurrent(q, k, v, g, beta, scale, S0, cu, None, None)
    assert all(np.all(x == 0) for x in grads)


def test_pure_decay_dh0():
    q, k, v, g, beta, scale, S0, cu, do, dht = rand_case(T=8, HV=1)
    beta = np.zeros_like(beta)
    *_, dh0 = BW.kda_backward_recurrent(q, k, v, g, beta, scale, S0, cu, None, dht)
    decay = np.exp(np.sum(g[0], axis=0))               # [HV, K]
    assert np.allclose(dh0[0], decay[:, :, None] * dht[0], rtol=1e-13)


# --------------------------------------------------------------------------- planted mistakes

SRC = inspect.getsource(BW.kda_backward_recurrent)
MUTANTS = {
    "dg from S_{t-1}": ("dg[t, j] = np.sum(dSp * sp, axis=1)",
                        "dg[t, j] = np.sum(dSp * sp / np.exp(gf[t, j])[:, None], axis=1)"),
    "dk without the residual path": ("dk[t, h] += bf[t, j] * (dS @ r) - sp @ dr",
                                     "dk[t, h] += bf[t, j] * (dS @ r)"),
    "dbeta with the wrong sign": ("db[t, j] = r @ dSk", "db[t, j] = -(r @ dSk)"),
    "no decay of dS": ("dS = np.exp(gf[t, j])[:, None] * dSp", "dS = dSp"),
    "dq from S'": ("dq[t, h] += scale * st @ dof[t, j]", "dq[t, h] += scale * sp @ dof[t, j]"),
    "dS' keeps the write": ("dSp = dS - np.outer(kf[t, h], dr)", "dSp = dS"),
}


def mutant(name):
    a, b = MUTANTS[name]
    assert SRC.count(a) == 1, name
    ns = dict(vars(BW))
    exec(SRC.replace(a, b), ns)
    return ns["kda_backward_recurrent"]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_backward_mistakes_are_caught(name):
    with pytest.raises(AssertionError):
        pin_finite_differences(mutant(name), rand_case(**CASES["dense_gva"]))


# --------------------------------------------------------------------------- the chunked form

from oracle.backward_chunked import kda_backward_chunked  # noqa: E402


@pytest.mark.parametrize("kw", [
    dict(B=1, T=40, H=1, HV=1, K=6, V=5),                      # ragged last chunk
    dict(B=2, T=16, H=1, HV=2, K=4, V=3),                      # one exact chunk, G = 2
    dict(H=2, HV=2, K=3, V=2, cu=np.array([0, 5, 5, 37])),     # varlen with an empty sequence
    dict(B=1, T=33, H=1, HV=1, K=5, V=4, h0=False),
], ids=["ragged", "gva", "varlen", "no_h0"])
def test_chunked_backward_equals_the_recurrence(kw):
    # the chunk-level reverse sweep (records, two chains, per-chunk local gradients) that the
    # GPU kernels follow gives the token recurrence's gradients
    case = rand_case(**kw)
    a = BW.kda_backward_recurrent(*case)
    b = kda_backward_chunked(*case)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), a, b):
        assert np.allclose(x, y, rtol=1e-10, atol=1e-12), name


def test_chunked_backward_without_dht():
    q, k, v, g, beta, scale, S0, cu, do, dht = rand_case(B=1, T=21, H=1, HV=1, K=4, V=3)
    a = BW.kda_backward_recurrent(q, k, v, g, beta, scale, S0, cu, do, None)
    b = kda_backward_chunked(q, k, v, g, beta, scale, S0, cu, do, None)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------- the C backward

def _c_bwd(q, k, v, g, beta, scale, S0, cu, do, dht):
    from oracle.native import kda_oracle_bwd_c
    return kda_oracle_bwd_c(q, k, v, g, beta, scale, S0, cu, do, dht, n_threads=2)


@pytest.mark.parametrize("name", list(CASES))
def test_c_backward_matches_finite_differences(name):
    # the C reverse recurrence against central differences of the fp64 forward (recurrent.py)
    pin_finite_differences(_c_bwd, rand_case(**CASES[name]))


def test_c_backward_checkpoint_segments_match_finite_differences():
    # 600 tokens: three 256-token checkpoint segments, the last one partial, and a sequence
    # boundary inside a segment
    cu = np.array([0, 300, 300, 600])
    pin_finite_differences(_c_bwd, rand_case(H=1, HV=2, K=3, V=2, cu=cu))


def _f32_case(case):
    # the C oracle reads fp32 carriers: round every input to fp32 first, so both oracles see
    # the same values
    r = lambda x: x if x is None or np.isscalar(x) else np.asarray(x, np.float32).astype(np.float64)
    q, k, v, g, beta, scale, S0, cu, do, dht = case
    return (r(q), r(k), r(v), r(g), r(beta), scale, r(S0), cu, r(do), r(dht))


@pytest.mark.parametrize("name", list(CASES))
def test_c_backward_agrees_with_python_backward(name):
    case = _f32_case(rand_case(**CASES[name]))
    a = _c_bwd(*case)
    b = BW.kda_backward_recurrent(*case)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, np.asarray(y).reshape(x.shape), rtol=1e-12, atol=1e-13)


def test_c_backward_decay_only_and_zero_loss():
    q, k, v, g, beta, scale, S0, cu, do, dht = _f32_case(rand_case(B=1, T=300, H=1, HV=1, K=3,
                                                                   V=2))
    beta0 = np.zeros_like(beta)
    *_, dh0 = _c_bwd(q, k, v, g, beta0, scale, S0, cu, np.zeros_like(do), dht)
    # beta = 0: final = exp(sum g) h0 per key row, so dh0 = exp(sum g) dht
    np.testing.assert_allclose(dh0, np.exp(g.sum(axis=1))[..., None] * dht, rtol=1e-12)
    grads = _c_bwd(q, k, v, g, beta, scale, S0, cu, np.zeros_like(do), np.zeros_like(dht))
    assert all(np.count_nonzero(x) == 0 for x in grads)
