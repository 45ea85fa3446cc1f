"""Write the stored expected values under tests/golden/ (calls only oracle/).

The pages print no worked example for the recurrence, so the stored values
come from the exact and high-precision forms in oracle/exact.py:

  rational_g0.json   exact rational results (fractions) for dyadic inputs with
                     zero log-decay (retention factor exactly 1), so the float
                     forms see the same inputs exactly; pins the delta-rule
                     algebra: erase against the state, write strength on the
                     prediction error, read after the write.
  mp50_decay.json    50-digit results with nonzero log-decays (some beyond the
                     -5 floor, so the clamp is exercised), stored to 25 digits.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import exact  # noqa: E402


def dyadic(rng, shape, bits=4, scale=1.0):
    return (np.round(rng.uniform(-scale, scale, shape) * 2 ** bits) / 2 ** bits).tolist()


def main():
    rng = np.random.default_rng(20260727)
    T, dk, dv = 6, 3, 2
    q = dyadic(rng, (T, dk))
    k = dyadic(rng, (T, dk), scale=0.75)
    v = dyadic(rng, (T, dv), scale=2.0)
    beta = (np.round(rng.uniform(0, 1, T) * 16) / 16).tolist()
    S0 = dyadic(rng, (dk, dv))
    ones = [[1] * dk for _ in range(T)]
    o, S = exact.seq_rational(q, k, v, ones, beta, S0)
    rec = {
        "what": "exact rational KDA recurrence, log-decay 0 (retention 1)",
        "source": "oracle.exact.seq_rational via tests/golden/make_golden.py",
        "shape": {"T": T, "dk": dk, "dv": dv},
        "q": q, "k": k, "v": v, "beta": beta, "g": [[0.0] * dk for _ in range(T)], "S0": S0,
        "o": [[str(x) for x in row] for row in o],
        "S_T": [[str(x) for x in row] for row in S],
    }
    with open(os.path.join(HERE, "rational_g0.json"), "w") as f:
        json.dump(rec, f, indent=1)

    rng = np.random.default_rng(20260804)
    T, dk, dv = 8, 4, 3
    f32 = lambda a: np.asarray(a, np.float32).tolist()
    q = f32(rng.standard_normal((T, dk)) / 2)
    k = f32(rng.standard_normal((T, dk)) / 2)
    v = f32(rng.standard_normal((T, dv)))
    beta = f32(rng.uniform(0, 1, T))
    g = rng.uniform(-7, 0.5, (T, dk))
    g = f32(g)
    S0 = f32(rng.standard_normal((dk, dv)))
    import mpmath
    with mpmath.workdps(60):
        om, Sm = exact.seq_mp(q, k, v, g, beta, S0, dps=50)
    # seq_mp returns floats; recompute at 50 digits keeping strings
    with mpmath.workdps(50):
        m = mpmath.mpf
        S = [[m(x) for x in row] for row in S0]
        outs = []
        for t in range(T):
            a = [mpmath.exp(min(max(m(x), m(-5)), m(0))) for x in g[t]]
            P = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
            u = [m(beta[t]) * (m(v[t][j]) - mpmath.fsum(P[i][j] * m(k[t][i]) for i in range(dk)))
                 for j in range(dv)]
            S = [[P[i][j] + m(k[t][i]) * u[j] for j in range(dv)] for i in range(dk)]
            outs.append([mpmath.fsum(S[i][j] * m(q[t][i]) for i in range(dk)) for j in range(dv)])
        o_s = [[mpmath.nstr(x, 25) for x in row] for row in outs]
        S_s = [[mpmath.nstr(x, 25) for x in row] for row in S]
    assert np.allclose(np.array(o_s, float), om, rtol=1e-14, atol=1e-300)
    rec = {
        "what": "KDA recurrence at 50 digits with log-decays in [-7, 0.5] (clamped to [-5, 0])",
        "source": "oracle.exact (mpmath) via tests/golden/make_golden.py",
        "shape": {"T": T, "dk": dk, "dv": dv},
        "q": q, "k": k, "v": v, "beta": beta, "g": g, "S0": S0,
        "o": o_s, "S_T": S_s,
    }
    with open(os.path.join(HERE, "mp50_decay.json"), "w") as f:
        json.dump(rec, f, indent=1)


if __name__ == "__main__":
    main()
