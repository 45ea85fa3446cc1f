"""Pins of the oracle's gate option: g read as raw gate logits x, with
per-channel log-decay -5 sigmoid(x) (a sigmoid scaled to the -5 floor; "Kimi K3
goes trillion-scale with sparse MoE efficiency" subtitles, cue 14 gives the
floor on retention, not the formula).

Each pin rests on something outside the oracle: SciPy's logistic function for
the closed form with beta = 0, the sequential NumPy recurrence fed with
SciPy-computed decays, and the exact limits of the sigmoid."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import c_oracle, ref

GATE = c_oracle.GATE_SIGMOID


def _inputs(rng, B, T, H, dk, dv, xscale=3.0):
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    x = (xscale * rng.standard_normal((B, T, H, dk))).astype(np.float32)
    beta = expit(rng.standard_normal((B, T, H))).astype(np.float32)
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, x, beta, S0


def test_beta_zero_closed_form_with_library_sigmoid():
    # beta = 0: S_t = Diag(exp(sum_{s<=t} -5 expit(x_s))) S0 and o_t = S_t^T q_t.
    # (9 tokens keep the decayed values far above any absolute tolerance)
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 9, 3, 8, 5
    q, k, v, x, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    beta[:] = 0
    o, ST = c_oracle.fwd(q, k, v, x, beta, S0=S0, gate=GATE)
    cum = np.cumsum(-5.0 * expit(x.astype(np.float64)), axis=1)       # [B,T,H,dk]
    St = np.exp(cum)[..., None] * S0[:, None]                         # [B,T,H,dk,dv]
    o_ref = np.einsum("bthkv,bthk->bthv", St, q.astype(np.float64))
    np.testing.assert_allclose(ST, St[:, -1], rtol=1e-12, atol=0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-14 * np.abs(o_ref).max())


def test_full_recurrence_matches_numpy_with_library_decays():
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 1, 41, 2, 6, 7
    q, k, v, x, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    o, ST = c_oracle.fwd(q, k, v, x, beta, S0=S0, gate=GATE)
    g = -5.0 * expit(x.astype(np.float64))
    for h in range(H):
        o_r, S_r = ref.seq(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], beta[0, :, h], S0[0, h])
        np.testing.assert_allclose(o[0, :, h], o_r, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ST[0, h], S_r, rtol=1e-11, atol=1e-12)


def test_sigmoid_limits_reach_the_bounds_exactly():
    # x -> +inf gives log-decay exactly -5 (the floor); x -> -inf gives 0
    # (no decay): the same results as log-decay inputs -5 and 0.
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 1, 19, 2, 4, 3
    q, k, v, _, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    sign = np.where(rng.random((B, T, H, dk)) < 0.5, 1.0, -1.0)
    x = (sign * 1e30).astype(np.float32)
    g = np.where(sign > 0, -5.0, 0.0).astype(np.float32)
    o1, S1 = c_oracle.fwd(q, k, v, x, beta, S0=S0, gate=GATE)
    o0, S0_ = c_oracle.fwd(q, k, v, g, beta, S0=S0)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(S1, S0_)


def test_zero_logit_is_half_the_floor():
    # sigmoid(0) = 1/2: log-decay -2.5 for every channel; beta = 0, q = e_0.
    B, T, H, dk, dv = 1, 3, 1, 2, 2
    q = np.zeros((B, T, H, dk), np.float32)
    q[..., 0] = 1
    k = np.zeros_like(q)
    v = np.zeros((B, T, H, dv), np.float32)
    x = np.zeros((B, T, H, dk), np.float32)
    beta = np.zeros((B, T, H), np.float32)
    S0 = np.ones((B, H, dk, dv))
    o, ST = c_oracle.fwd(q, k, v, x, beta, S0=S0, gate=GATE)
    for t in range(T):
        np.testing.assert_allclose(o[0, t, 0], np.exp(-2.5 * (t + 1)), rtol=1e-15)
    np.testing.assert_allclose(ST[0, 0], np.exp(-7.5), rtol=1e-15)


def test_nan_logit_propagates_from_its_token_on():
    # NaN in one channel's logit poisons that row of the decayed state, and the
    # erase term P^T k (NaN * 0 is NaN) carries it into every column; outputs
    # before that token stay finite.
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 1, 5, 1, 4, 3
    q, k, v, x, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    x[0, 2, 0, 1] = np.nan
    o, ST = c_oracle.fwd(q, k, v, x, beta, S0=S0, gate=GATE)
    assert np.isfinite(o[0, :2]).all()
    assert np.isnan(o[0, 2:]).all() and np.isnan(ST).all()


@pytest.mark.parametrize("mistake", ["no_scale", "plus_sign", "flipped_logit", "softplus"])
def test_gate_pin_rejects_plausible_mistakes(mistake):
    # A gate written wrongly in a copy of the closed form fails the pin above.
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 9, 3, 8, 5
    q, k, v, x, beta, S0 = _inputs(rng, B, T, H, dk, dv)
    beta[:] = 0
    _, ST = c_oracle.fwd(q, k, v, x, beta, S0=S0, gate=GATE)
    xd = x.astype(np.float64)
    wrong = {"no_scale": -expit(xd), "plus_sign": np.minimum(5.0 * expit(xd), 0.0),
             "flipped_logit": -5.0 * expit(-xd),
             "softplus": np.maximum(-np.logaddexp(0.0, xd), -5.0)}[mistake]
    St = np.exp(np.cumsum(wrong, axis=1))[..., None] * S0[:, None]
    assert not np.allclose(ST, St[:, -1], rtol=1e-6, atol=0)
