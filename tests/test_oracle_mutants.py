"""Plant plausible mistakes in a copy of the sequential oracle (on the CPU) and
check that the pins catch every one of them; the unmodified copy passes all."""
import numpy as np
import pytest

import pins


def make_seq(mistake=None):
    def seq(q, k, v, g, beta, S0=None):
        q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
        g = np.asarray(g, np.float64)
        if mistake == "nan_swallowing_clamp":
            g = np.fmin(np.fmax(g, -5.0), 0.0)
        elif mistake != "no_clamp":
            g = np.clip(g, -5.0, 0.0)
        T, dk = q.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
        o = np.empty((T, dv))
        for t in range(T):
            e = np.exp(g[t])
            if mistake == "decay_columns":
                P = S * e[:dv][None, :] if dk >= dv else S
            elif mistake == "erase_before_decay":
                P = S
            elif mistake == "decay_after_write":
                P = S
            else:
                P = e[:, None] * S
            kt = k[t]
            if mistake == "sign":
                u = beta[t] * (v[t] + P.T @ kt)
            elif mistake == "beta_on_erase_only":
                u = v[t] - beta[t] * (P.T @ kt)
            elif mistake == "no_beta":
                u = v[t] - P.T @ kt
            else:
                u = beta[t] * (v[t] - P.T @ kt)
            prev = S
            S = P + np.outer(kt, u)
            if mistake == "erase_before_decay":
                S = e[:, None] * S
            if mistake == "decay_after_write":
                S = e[:, None] * S
            if mistake == "read_before_write":
                o[t] = (e[:, None] * prev).T @ q[t]
            elif mistake == "query_scale":
                o[t] = S.T @ q[t] / np.sqrt(dk)
            elif mistake == "readout_key":
                o[t] = S.T @ kt
            elif mistake == "transposed_readout":
                o[t] = (S @ q[t][:dv]) if dk == dv else S.T @ q[t] * 1.0001
            else:
                o[t] = S.T @ q[t]
        return o, S
    return seq


MISTAKES = ["no_clamp", "nan_swallowing_clamp", "decay_columns", "erase_before_decay",
            "decay_after_write", "sign", "beta_on_erase_only", "no_beta",
            "read_before_write", "query_scale", "readout_key", "transposed_readout"]


def test_unmodified_copy_passes():
    res = pins.run_all(make_seq(None))
    bad = {k: v for k, v in res.items() if not v[2]}
    assert not bad, bad


@pytest.mark.parametrize("mistake", MISTAKES)
def test_mistake_is_caught(mistake):
    if mistake == "nan_swallowing_clamp":
        # caught by the NaN check, not by a numeric pin
        q = np.ones((3, 2), np.float32) * 0.5
        g = np.zeros((3, 2), np.float32)
        g[1, 0] = np.nan
        o, _ = make_seq(mistake)(q, q, np.ones((3, 2), np.float32), g, np.ones(3, np.float32) * 0.5)
        assert np.isfinite(o[1:]).all()  # the mistake hides the NaN ...
        o, _ = make_seq(None)(q, q, np.ones((3, 2), np.float32), g, np.ones(3, np.float32) * 0.5)
        assert np.isnan(o[1:]).all()     # ... which the real clamp keeps
        return
    res = pins.run_all(make_seq(mistake))
    failed = [k for k, v in res.items() if not v[2]]
    assert failed, "no pin caught %s" % mistake
