"""The KDA token recurrence in exact rational arithmetic (test infrastructure).

For tiny inputs whose decays are given as rationals a = exp(g) (so g = ln a), every step of the
recurrence in recurrent.py is a rational operation, and fractions.Fraction evaluates it with no
rounding at all. Comparing the fp64 oracle against this pins its rounding behaviour (it must
agree to a few ulps of the result) independently of any floating-point library.

Same step order as recurrent.py (decay, residual, write, then read), which follows "手撕KDA"
("KDA by hand"), section 1.
"""
from __future__ import annotations

from fractions import Fraction


def kda_exact(q, k, v, a, beta, scale, S0=None):
    """One sequence, one head. q, k: [T][K]; v: [T][V]; a: [T][K] decay factors exp(g);
    beta: [T]; scale: Fraction; S0: [K][V] or None. All entries Fractions (or ints).
    Returns (o [T][V], S [K][V]) as Fractions."""
    T = len(q)
    K = len(q[0])
    V = len(v[0])
    S = [[Fraction(0)] * V for _ in range(K)] if S0 is None else \
        [[Fraction(x) for x in row] for row in S0]
    o = []
    for t in range(T):
        for d in range(K):
            for n in range(V):
                S[d][n] *= a[t][d]
        r = [v[t][n] - sum(S[d][n] * k[t][d] for d in range(K)) for n in range(V)]
        for d in range(K):
            for n in range(V):
                S[d][n] += beta[t] * k[t][d] * r[n]
        o.append([scale * sum(S[d][n] * q[t][d] for d in range(K)) for n in range(V)])
    return o, S
