"""Exact and high-precision forms of the sequential KDA recurrence.

Test infrastructure only. These restate the per-token definition
(P = Diag(a) S with a = e^g per key channel; u = beta (v - P^T k);
S = P + k u^T; o = S^T q) in arithmetic that does not round (fractions) or
rounds far below double precision (mpmath), to pin the fp64 oracles.
Arrays are nested lists per (batch, head): q, k [T][dk], v [T][dv],
beta [T], decay [T][dk], S0 [dk][dv].
"""
from fractions import Fraction

import mpmath


def seq_rational(q, k, v, decay, beta, S0=None):
    """Exact recurrence with the per-channel retention factors a = e^g given
    directly as rationals (so no exponential is evaluated)."""
    T, dk, dv = len(q), len(q[0]), len(v[0])
    F = Fraction
    S = [[F(0)] * dv for _ in range(dk)] if S0 is None else [[F(x) for x in row] for row in S0]
    out = []
    for t in range(T):
        a = [F(x) for x in decay[t]]
        kt = [F(x) for x in k[t]]
        qt = [F(x) for x in q[t]]
        bt = F(beta[t])
        P = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
        u = [bt * (F(v[t][j]) - sum(P[i][j] * kt[i] for i in range(dk))) for j in range(dv)]
        S = [[P[i][j] + kt[i] * u[j] for j in range(dv)] for i in range(dk)]
        out.append([sum(S[i][j] * qt[i] for i in range(dk)) for j in range(dv)])
    return out, S


def seq_mp(q, k, v, g, beta, S0=None, dps=50):
    """Recurrence with log-decays g (clamped to [-5, 0]) at `dps` decimal digits.
    Float inputs are converted exactly (mpf of a binary float is exact)."""
    with mpmath.workdps(dps):
        m = mpmath.mpf
        T, dk, dv = len(q), len(q[0]), len(v[0])
        S = [[m(0)] * dv for _ in range(dk)] if S0 is None else [[m(float(x)) for x in row] for row in S0]
        out = []
        for t in range(T):
            gl = [min(max(m(float(x)), m(-5)), m(0)) for x in g[t]]
            a = [mpmath.exp(x) for x in gl]
            kt = [m(float(x)) for x in k[t]]
            qt = [m(float(x)) for x in q[t]]
            bt = m(float(beta[t]))
            P = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
            u = [bt * (m(float(v[t][j])) - mpmath.fsum(P[i][j] * kt[i] for i in range(dk)))
                 for j in range(dv)]
            S = [[P[i][j] + kt[i] * u[j] for j in range(dv)] for i in range(dk)]
            out.append([mpmath.fsum(S[i][j] * qt[i] for i in range(dk)) for j in range(dv)])
        return [[float(x) for x in row] for row in out], [[float(x) for x in row] for row in S]
