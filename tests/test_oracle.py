"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is a function of an implementation ``impl(q, k, v, g, beta, scale, h0, cu) ->
(o, final)`` so that the same checks run on the oracle (must pass) and on deliberately broken
copies of the recurrence planted below (each must fail at least one pin). The pins are:

  golden      hand-worked tiny cases in tests/golden/ (exact rationals, derivation included)
  P-1         one token: closed form
  P-2         K = V = 1: scalar closed form  s_t = a_t s_{t-1} (1 - b_t k_t^2) + b_t k_t v_t
  P-3         beta = 0: pure decay, o_t = scale (q_t * exp(sum_{tau<=t} g))^T S0
  P-4         g = 0, beta = 1, one fixed unit key k = q: o_t = scale v_t exactly and
              S_T = (I - k k^T) S0 + k v_T^T (plain delta rule / DeltaNet retrieval)
  P-5         linearity in (v, h0) jointly
  P-6         chunked (WY) form == recurrence for chunk sizes 1..64, ragged tails
  P-7         Neumann inverse == forward substitution == LAPACK; nilpotency L^16 = 0
  P-8         state passing: run(T1 + T2) == run(T2, h0 = final(T1))
  P-9         varlen == per-sequence runs; grouped value heads == repeated q/k
  P-10        exact rational arithmetic (fractions) on tiny inputs
  C oracle    == numpy recurrence to ~1e-12
"""
from __future__ import annotations

import glob
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle.chunked import (chunk_prepare, inverse_forward_substitution, inverse_neumann,
                            kda_chunked)
from oracle.exact import kda_exact
from oracle.native import kda_oracle_c
from oracle.recurrent import kda_recurrent

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


# --------------------------------------------------------------------------- implementations

def impl_recurrent(q, k, v, g, beta, scale, h0=None, cu=None):
    return kda_recurrent(q, k, v, g, beta, scale, h0, cu)


def impl_c(q, k, v, g, beta, scale, h0=None, cu=None):
    return kda_oracle_c(q, k, v, g, beta, scale, h0, cu, n_threads=2)


def impl_chunked16(q, k, v, g, beta, scale, h0=None, cu=None):
    return kda_chunked(q, k, v, g, beta, scale, h0, cu, C=16)


def impl_chunked3(q, k, v, g, beta, scale, h0=None, cu=None):
    return kda_chunked(q, k, v, g, beta, scale, h0, cu, C=3)


ORACLES = {"recurrent": impl_recurrent, "c": impl_c, "chunked16": impl_chunked16,
           "chunked3": impl_chunked3}


def mutant(kind):
    """A copy of the recurrence with one planted mistake (test-only, CPU)."""

    def impl(q, k, v, g, beta, scale, h0=None, cu=None):
        q, k, v, g, beta = [np.asarray(x, np.float64) for x in (q, k, v, g, beta)]
        B, T, H, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        G = HV // H
        bounds = [(b * T, (b + 1) * T) for b in range(B)] if cu is None else \
            [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
        qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
        vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV, K), beta.reshape(B * T, HV)
        o = np.zeros((B * T, HV, V))
        fin = np.zeros((len(bounds), HV, K, V))
        hq = np.arange(HV) % H if kind == "gva_mod" else np.arange(HV) // G
        sc = 1.0 if kind == "no_scale" else scale
        for s, (bos, eos) in enumerate(bounds):
            S = np.zeros((HV, K, V)) if h0 is None else np.array(h0[s], np.float64)
            for t in range(bos, eos):
                kt, qt = kf[t][hq], qf[t][hq]
                dec = np.exp(gf[t])[:, :, None]
                if kind == "read_before_write":
                    o[t] = sc * np.einsum('jkv,jk->jv', S * dec, qt)
                if kind not in ("no_decay", "decay_after_write"):
                    S = S * dec
                if kind == "transposed_read":
                    r = vf[t] - np.einsum('jkv,jv->jk', S, kt)
                elif kind == "residual_before_decay":
                    r = vf[t] - np.einsum('jkv,jk->jv', S / dec, kt)
                else:
                    r = vf[t] - np.einsum('jkv,jk->jv', S, kt)
                if kind == "residual_sign":
                    r = vf[t] + np.einsum('jkv,jk->jv', S, kt)
                bt = np.ones_like(bf[t]) if kind == "beta_dropped" else bf[t]
                S = S + bt[:, None, None] * kt[:, :, None] * r[:, None, :]
                if kind == "decay_after_write":
                    S = S * dec
                if kind != "read_before_write":
                    o[t] = sc * np.einsum('jkv,jk->jv', S, qt)
            fin[s] = S
        return o.reshape(B, T, HV, V), fin

    return impl


MUTANTS = ["no_decay", "decay_after_write", "read_before_write", "residual_sign",
           "transposed_read", "residual_before_decay", "beta_dropped", "gva_mod", "no_scale"]


# --------------------------------------------------------------------------- input helpers

def rand_case(B=1, T=23, H=2, HV=4, K=5, V=3, h0=True, glo=-0.6):
    q = RNG.standard_normal((B, T, H, K)) / np.sqrt(K)
    k = RNG.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = RNG.standard_normal((B, T, HV, V))
    g = RNG.uniform(glo, 0.0, (B, T, HV, K))
    beta = RNG.uniform(0.05, 0.95, (B, T, HV))
    S0 = RNG.standard_normal((B, HV, K, V)) * 0.5 if h0 else None
    return q, k, v, g, beta, K ** -0.5, S0


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------- pins

def _frac(x):
    return Fraction(x)


def _load_golden():
    cases = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        with open(path) as f:
            cases.append((os.path.basename(path), json.load(f)))
    return cases


def pin_golden(impl):
    worst = 0.0
    for _, c in _load_golden():
        tof = lambda x: np.vectorize(lambda s: float(Fraction(s)))(np.array(x, dtype=object))
        q, k, v = tof(c["q"])[None], tof(c["k"])[None], tof(c["v"])[None]
        a = tof(c["a"])[None]
        beta = tof(c["beta"])[None]
        h0 = None if c["h0"] is None else tof(c["h0"])
        o, fin = impl(q, k, v, np.log(a), beta, float(Fraction(c["scale"])), h0, None)
        worst = max(worst, relerr(o[0], tof(c["o"])), relerr(fin, tof(c["final"])))
    return worst


def pin_single_token(impl):
    q, k, v, g, beta, scale, S0 = rand_case(T=1, H=1, HV=1, K=5, V=5)   # square: a transposed
    # state read gives a different (not just mis-shaped) answer
    o, fin = impl(q, k, v, g, beta, scale, S0, None)
    Sd = np.exp(g[0, 0, 0])[:, None] * S0[0, 0]                 # diag(e^g) S0
    kk = k[0, 0, 0]
    S1 = Sd + beta[0, 0, 0] * np.outer(kk, v[0, 0, 0] - Sd.T @ kk)
    return max(relerr(fin[0, 0], S1), relerr(o[0, 0, 0], scale * S1.T @ q[0, 0, 0]))


def pin_scalar(impl):
    T = 17
    q = RNG.standard_normal((1, T, 1, 1))
    k = RNG.uniform(-1, 1, (1, T, 1, 1))
    v = RNG.standard_normal((1, T, 1, 1))
    g = RNG.uniform(-1, 0, (1, T, 1, 1))
    beta = RNG.uniform(0, 1, (1, T, 1))
    s = 0.7
    ref_o = []
    for t in range(T):
        a, kt, bt = np.exp(g[0, t, 0, 0]), k[0, t, 0, 0], beta[0, t, 0]
        s = a * s * (1 - bt * kt * kt) + bt * kt * v[0, t, 0, 0]
        ref_o.append(0.3 * q[0, t, 0, 0] * s)
    o, fin = impl(q, k, v, g, beta, 0.3, np.full((1, 1, 1, 1), 0.7), None)
    return max(relerr(o.ravel(), ref_o), relerr(fin.ravel(), [s]))


def pin_beta_zero(impl):
    q, k, v, g, beta, scale, S0 = rand_case(T=19, H=2, HV=2, K=4, V=3)
    beta = np.zeros_like(beta)
    o, fin = impl(q, k, v, g, beta, scale, S0, None)
    cum = np.cumsum(g[0], axis=0)                                  # [T, HV, K]
    ref_o = scale * np.einsum('tjk,jkv->tjv', q[0] * np.exp(cum), S0[0])
    ref_f = np.exp(cum[-1])[:, :, None] * S0[0]
    return max(relerr(o[0], ref_o), relerr(fin[0], ref_f))


def pin_deltanet_unit_key(impl):
    T, K, V = 13, 5, 3
    kvec = RNG.standard_normal(K)
    kvec /= np.linalg.norm(kvec)
    k = np.broadcast_to(kvec, (1, T, 1, K)).copy()
    q = k.copy()
    v = RNG.standard_normal((1, T, 1, V))
    g = np.zeros((1, T, 1, K))
    beta = np.ones((1, T, 1))
    S0 = RNG.standard_normal((1, 1, K, V))
    o, fin = impl(q, k, v, g, beta, 0.25, S0, None)
    ref_f = (np.eye(K) - np.outer(kvec, kvec)) @ S0[0, 0] + np.outer(kvec, v[0, -1, 0])
    return max(relerr(o[0, :, 0], 0.25 * v[0, :, 0]), relerr(fin[0, 0], ref_f))


def pin_linearity(impl):
    q, k, v, g, beta, scale, S0 = rand_case(T=21, H=1, HV=2, K=4, V=4)
    v2 = RNG.standard_normal(v.shape)
    S02 = RNG.standard_normal(S0.shape)
    c = -1.7
    o1, f1 = impl(q, k, v, g, beta, scale, S0, None)
    o2, f2 = impl(q, k, v2, g, beta, scale, S02, None)
    o3, f3 = impl(q, k, v + c * v2, g, beta, scale, S0 + c * S02, None)
    return max(relerr(o3, o1 + c * o2), relerr(f3, f1 + c * f2))


def pin_state_passing(impl):
    q, k, v, g, beta, scale, S0 = rand_case(T=40, H=1, HV=2, K=4, V=3)
    o, fin = impl(q, k, v, g, beta, scale, S0, None)
    T1 = 17
    sl = lambda x, a, b: x[:, a:b]
    oa, fa = impl(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(g, 0, T1), sl(beta, 0, T1),
                  scale, S0, None)
    ob, fb = impl(sl(q, T1, 40), sl(k, T1, 40), sl(v, T1, 40), sl(g, T1, 40),
                  sl(beta, T1, 40), scale, fa, None)
    return max(relerr(np.concatenate([oa, ob], 1), o), relerr(fb, fin))


def pin_varlen(impl):
    lens = [7, 0, 16, 33]
    T = sum(lens)
    q, k, v, g, beta, scale, _ = rand_case(T=T, H=1, HV=2, K=4, V=3)
    S0 = RNG.standard_normal((len(lens), 2, 4, 3))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    o, fin = impl(q, k, v, g, beta, scale, S0, cu)
    worst = 0.0
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            worst = max(worst, relerr(fin[s], S0[s]))
            continue
        os_, fs = impl(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], scale,
                       S0[s:s + 1], None)
        worst = max(worst, relerr(o[:, a:b], os_), relerr(fin[s], fs[0]))
    return worst


def pin_gva(impl):
    q, k, v, g, beta, scale, S0 = rand_case(T=14, H=2, HV=6, K=4, V=3)
    o, fin = impl(q, k, v, g, beta, scale, S0, None)
    G = 3
    qr, kr = np.repeat(q, G, axis=2), np.repeat(k, G, axis=2)     # repeat_interleave
    o2, f2 = impl(qr, kr, v, g, beta, scale, S0, None)
    return max(relerr(o, o2), relerr(fin, f2))


def pin_exact(impl):
    rng = np.random.default_rng(7)
    worst = 0.0
    for (T, K, V) in [(1, 1, 1), (3, 2, 2), (6, 3, 2), (5, 1, 3)]:
        rat = lambda lo, hi: Fraction(int(rng.integers(lo, hi)), 8)
        q = [[rat(-8, 9) for _ in range(K)] for _ in range(T)]
        k = [[rat(-8, 9) for _ in range(K)] for _ in range(T)]
        v = [[rat(-16, 17) for _ in range(V)] for _ in range(T)]
        a = [[Fraction(int(rng.integers(1, 17)), 16) for _ in range(K)] for _ in range(T)]
        b = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
        S0 = [[rat(-8, 9) for _ in range(V)] for _ in range(K)]
        scale = Fraction(1, 2)
        oe, Se = kda_exact(q, k, v, a, b, scale, S0)
        f = lambda x: np.array([[float(y) for y in row] for row in x])
        o, fin = impl(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                      np.log(f(a))[None, :, None], np.array([float(x) for x in b])[None, :, None],
                      0.5, f(S0)[None, None], None)
        worst = max(worst, relerr(o[0, :, 0], f(oe)), relerr(fin[0, 0], f(Se)))
    return worst


PINS = {
    "golden": (pin_golden, 1e-14),
    "single_token": (pin_single_token, 1e-13),
    "scalar": (pin_scalar, 1e-12),
    "beta_zero": (pin_beta_zero, 1e-13),
    "deltanet_unit_key": (pin_deltanet_unit_key, 1e-12),
    "linearity": (pin_linearity, 1e-12),
    "state_passing": (pin_state_passing, 1e-12),
    "varlen": (pin_varlen, 1e-12),
    "gva": (pin_gva, 1e-13),
    "exact": (pin_exact, 1e-13),
}


@pytest.mark.parametrize("oracle", list(ORACLES))
@pytest.mark.parametrize("pin", list(PINS))
def test_oracle_pins(oracle, pin):
    fn, tol = PINS[pin]
    if oracle == "c":
        # the C oracle takes fp32 inputs (exact carriers of what the GPU reads); the pins'
        # fp64 inputs (3/5, log(1/2), ...) are rounded on the way in, ~1e-7 relative. Its
        # exact agreement with the numpy recurrence is checked on fp32-exact inputs below.
        tol = max(tol, 2e-6)
    err = fn(ORACLES[oracle])
    assert err <= tol, f"{oracle} fails pin {pin}: rel err {err:.3e} > {tol}"


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind):
    impl = mutant(kind)

    def err_of(fn):
        try:
            return fn(impl)
        except (ValueError, IndexError):       # a shape mismatch is a failed pin too
            return float("inf")

    failed = [name for name, (fn, tol) in PINS.items() if not err_of(fn) <= tol * 10]
    assert failed, f"planted mistake '{kind}' passed every pin"


def test_mutant_harness_is_faithful():
    # the unbroken copy of the mutant harness passes every pin (so failures above come from
    # the planted mistake, not from the harness)
    impl = mutant("none")
    for name, (fn, tol) in PINS.items():
        assert fn(impl) <= tol, name


# --------------------------------------------------------------------------- P-6 chunked

@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64])
def test_chunked_equals_recurrent(C):
    q, k, v, g, beta, scale, S0 = rand_case(B=2, T=45, H=2, HV=4, K=6, V=5, glo=-0.4)
    o1, f1 = kda_recurrent(q, k, v, g, beta, scale, S0)
    o2, f2 = kda_chunked(q, k, v, g, beta, scale, S0, C=C)
    assert relerr(o2, o1) < 1e-12 and relerr(f2, f1) < 1e-12


def test_chunked_strong_decay_and_tail():
    # strong decay (log U(0.5, 0.9999)-like) and a tail chunk of 3 tokens
    q, k, v, g, beta, scale, S0 = rand_case(T=35, H=1, HV=1, K=8, V=4, glo=-0.69)
    o1, f1 = kda_recurrent(q, k, v, g, beta, scale, S0)
    o2, f2 = kda_chunked(q, k, v, g, beta, scale, S0, C=16)
    assert relerr(o2, o1) < 1e-12 and relerr(f2, f1) < 1e-12


# --------------------------------------------------------------------------- P-7 inverse

def _random_L(n=16, mag=0.3):
    L = np.tril(RNG.standard_normal((n, n)) * mag, -1)
    return L


def test_inverse_nilpotent_and_methods_agree():
    for _ in range(20):
        L = _random_L()
        assert np.array_equal(np.linalg.matrix_power(L, 16), np.zeros((16, 16))) or \
            np.abs(np.linalg.matrix_power(L, 16)).max() == 0.0
        X1 = inverse_forward_substitution(L)
        X2 = inverse_neumann(L)
        X3 = np.linalg.inv(np.eye(16) + L)
        X4 = scipy.linalg.solve_triangular(np.eye(16) + L, np.eye(16), lower=True,
                                           unit_diagonal=True)
        ref = np.abs(X3).max()
        assert np.abs(X1 - X3).max() < 1e-13 * ref
        assert np.abs(X2 - X3).max() < 1e-13 * ref
        assert np.abs(X4 - X3).max() < 1e-13 * ref
        assert np.abs((np.eye(16) + L) @ X2 - np.eye(16)).max() < 1e-13 * ref


def test_neumann_other_sizes():
    for n in (1, 2, 3, 5, 8, 17, 32):
        L = _random_L(n, 0.4)
        assert np.allclose(inverse_neumann(L), np.linalg.inv(np.eye(n) + L), rtol=0,
                           atol=1e-12 * max(1, np.abs(np.linalg.inv(np.eye(n) + L)).max()))


def test_chunk_prepare_identities():
    # (I + L) A = diag(beta); w and u solve the chunk's linear system; kr, qd, Mqk factorise
    q, k, v, g, beta, scale, _ = rand_case(T=37, H=1, HV=1, K=6, V=4)
    p = chunk_prepare(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], scale, 16)
    C = 16
    for c in range(p['A'].shape[0]):
        bvec = np.concatenate([beta[0, :, 0], np.zeros(48 - 37)])[16 * c:16 * c + 16]
        assert np.allclose((np.eye(C) + p['L'][c]) @ p['A'][c], np.diag(bvec), atol=1e-13)
        Gam = p['Gam'][c]
        kk = np.concatenate([k[0, :, 0], np.zeros((48 - 37, 6))])[16 * c:16 * c + 16]
        qq = np.concatenate([q[0, :, 0], np.zeros((48 - 37, 6))])[16 * c:16 * c + 16]
        # factorised forms (what a kernel evaluates) agree with the difference-exponent forms
        Lf = np.tril((kk * np.exp(Gam)) @ (kk * np.exp(-Gam)).T, -1) * bvec[:, None]
        Mf = np.tril(scale * (qq * np.exp(Gam)) @ (kk * np.exp(-Gam)).T)
        assert np.allclose(Lf, p['L'][c], atol=1e-13)
        assert np.allclose(Mf, p['Mqk'][c], atol=1e-13)
    assert list(p['n_valid']) == [16, 16, 5]


# --------------------------------------------------------------------------- C oracle

def test_c_oracle_matches_numpy_and_samples():
    q, k, v, g, beta, scale, _ = rand_case(B=1, T=70, H=2, HV=4, K=16, V=8)
    lens = [30, 0, 40]
    cu = np.array([0, 30, 30, 70], np.int64)
    S0 = RNG.standard_normal((3, 4, 16, 8))
    f32 = lambda x: x.astype(np.float32).astype(np.float64)
    args = [f32(x) for x in (q, k, v, g, beta)]
    o1, f1 = kda_recurrent(*args, scale, f32(S0), cu)
    o2, f2 = kda_oracle_c(*args, scale, f32(S0), cu, n_threads=3)
    assert relerr(o2, o1) < 1e-13 and relerr(f2, f1) < 1e-13
    units = [(2, 3), (0, 1)]
    o3, f3 = kda_oracle_c(*args, scale, f32(S0), cu, units=units, n_threads=2)
    assert np.array_equal(f3[2, 3], f2[2, 3]) and np.array_equal(f3[0, 1], f2[0, 1])
    assert np.all(f3[1] == 0) and np.array_equal(o3[0, 30:70, 3], o2[0, 30:70, 3])
    del lens


def test_state_affine_in_a_segment_start():
    # The decomposition the 32-token path's two-segment state pass relies on, checked on the
    # fp64 recurrence itself: a sequence's later segment run from a start state S_A equals the
    # run from zero plus y S_A (outputs) and phi S_A (final state), where y and phi are the
    # outputs and final state of the same tokens run with v = 0 from the identity (K columns).
    rng = np.random.default_rng(21)
    T, T_A, H, HV, K, V = 70, 29, 1, 2, 16, 8
    q = rng.standard_normal((1, T, H, K)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, T, H, K)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, HV, V))
    g = np.log(rng.uniform(0.8, 0.999, (1, T, HV, K)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, T, HV))))
    h0 = 0.1 * rng.standard_normal((1, HV, K, V))
    o, fin = kda_recurrent(q, k, v, g, beta, initial_state=h0)
    seg = lambda x, a, b: x[:, a:b]
    _, S_A = kda_recurrent(*(seg(x, 0, T_A) for x in (q, k, v, g, beta)), initial_state=h0)
    b = [seg(x, T_A, T) for x in (q, k, v, g, beta)]
    o0, S0 = kda_recurrent(*b)
    eye = np.broadcast_to(np.eye(K), (1, HV, K, K)).copy()
    y, phi = kda_recurrent(b[0], b[1], np.zeros((1, T - T_A, HV, K)), b[3], b[4],
                           initial_state=eye)
    o_b = o0 + np.einsum("btjk,jkv->btjv", y, S_A[0])
    fin_b = S0 + np.einsum("njkl,njlv->njkv", phi, S_A)
    assert np.allclose(o_b, o[:, T_A:], rtol=1e-11, atol=1e-12)
    assert np.allclose(fin_b, fin, rtol=1e-11, atol=1e-12)
    # the transition is not trivial here: S_A changes the later outputs
    assert np.abs(np.einsum("btjk,jkv->btjv", y, S_A[0])).max() > 1e-3
