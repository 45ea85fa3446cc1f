"""The fp64 oracle against what the definition fixes (CPU only).

The oracle forms (C sequential, NumPy sequential, NumPy chunked) are pinned by
closed forms, invariants, special cases and exact / 50-digit stored results;
see tests/pins.py for the statements and their sources on the pages.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import pins
from oracle import c_oracle, ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def c_fwd(q, k, v, g, beta, S0):
    """Per-(b,h) view of the C oracle."""
    o, S = c_oracle.fwd(q[None, :, None], k[None, :, None], v[None, :, None],
                        g[None, :, None], beta[None, :, None],
                        None if S0 is None else np.asarray(S0, np.float64)[None, None],
                        nthreads=1)
    return o[0, :, 0], S[0, 0]


FORMS = {"numpy_seq": ref.seq, "numpy_chunked": ref.chunked, "c_seq": c_fwd}


@pytest.mark.parametrize("form", sorted(FORMS))
@pytest.mark.parametrize("pin", [p[0] for p in pins.PINS])
def test_pin(form, pin):
    fn, tol = {n: (f, t) for n, f, t in pins.PINS}[pin]
    dev = fn(FORMS[form], np.random.default_rng(11))
    assert dev <= tol, "%s on %s deviates by %g (tolerance %g)" % (pin, form, dev, tol)


def test_bf16_range_bound():
    """The reciprocal decay over a 16-token tile at the -5 floor, e^(5*16), is
    below the bf16 maximum, and e^-80 is above the smallest normal bf16/fp32
    ("K3 tech report" transcript: the -5 bound keeps the 16-token reciprocal
    scaling under the bf16 limit). A 17-token tile still fits, 18 does not."""
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    min_normal = 2.0 ** -126
    assert math.exp(5 * 16) < bf16_max
    assert math.exp(-5 * 16) > min_normal
    assert math.exp(5 * 17) < bf16_max < math.exp(5 * 18)
    # fp16 (max 65504) would allow only two tokens at the floor
    assert math.exp(5 * 2) < 65504 < math.exp(5 * 3)


@pytest.mark.parametrize("form", sorted(FORMS))
def test_rational_fixture(form):
    rec = json.load(open(os.path.join(GOLDEN, "rational_g0.json")))
    arr = lambda key: np.array(rec[key], np.float32)
    o, S = FORMS[form](arr("q"), arr("k"), arr("v"), arr("g"), arr("beta"), arr("S0"))
    o_ex = np.array([[float(Fraction(x)) for x in r] for r in rec["o"]])
    S_ex = np.array([[float(Fraction(x)) for x in r] for r in rec["S_T"]])
    np.testing.assert_allclose(o, o_ex, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, S_ex, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("form", sorted(FORMS))
def test_mp50_fixture(form):
    rec = json.load(open(os.path.join(GOLDEN, "mp50_decay.json")))
    arr = lambda key: np.array(rec[key], np.float32)
    o, S = FORMS[form](arr("q"), arr("k"), arr("v"), arr("g"), arr("beta"), arr("S0"))
    np.testing.assert_allclose(o, np.array(rec["o"], float), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, np.array(rec["S_T"], float), rtol=1e-12, atol=1e-13)


def _batch(rng, B, T, H, dk, dv, s0=True):
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-rng.random((B, T, H, dk)) * 6).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


def test_c_matches_numpy_batched_and_threads():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = _batch(rng, 2, 29, 3, 6, 4)
    o_ref, S_ref = ref.seq_batched(q, k, v, g, beta, S0)
    for nt in (1, 3, 8):
        o, S = c_oracle.fwd(q, k, v, g, beta, S0, nthreads=nt)
        np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(S, S_ref, rtol=1e-13, atol=1e-14)


def test_c_bf16_inputs_widen_exactly():
    """bf16 bit patterns are widened exactly: same result as the float32 values
    they encode."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = _batch(rng, 1, 17, 2, 5, 3)
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    back = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    qb, kb, vb, gb, bb = (bits(x) for x in (q, k, v, g, beta))
    o1, S1 = c_oracle.fwd(qb, kb, vb, gb, bb, S0)
    o2, S2 = c_oracle.fwd(back(qb), back(kb), back(vb), back(gb), back(bb), S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_c_columns_subset():
    """The value-column-subset form equals the same columns of the full run."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = _batch(rng, 2, 23, 3, 6, 7)
    o, S = c_oracle.fwd(q, k, v, g, beta, S0)
    cols = [6, 0, 3]
    oc, Sc = c_oracle.fwd_cols(q, k, v, g, beta, 1, 2, cols, S0[1, 2][:, cols])
    np.testing.assert_allclose(oc, o[1, :, 2][:, cols], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Sc, S[1, 2][:, cols], rtol=1e-14, atol=1e-15)


def test_nan_propagates():
    """A NaN log-decay is not swallowed by the floor: the state row it touches
    becomes NaN and so does every later output."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, S0 = _batch(rng, 1, 10, 1, 4, 3)
    g[0, 4, 0, 2] = np.nan
    for o, S in (c_oracle.fwd(q, k, v, g, beta, S0),
                 ref.seq_batched(q, k, v, g, beta, S0)):
        assert np.isfinite(o[0, :4]).all()
        assert np.isnan(o[0, 4:]).all()
        assert np.isnan(S).any()


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(8)
    q, k, v, g, beta, S0 = _batch(rng, 1, 0, 2, 4, 3)
    o, S = c_oracle.fwd(q, k, v, g, beta, S0)
    assert o.shape == (1, 0, 2, 3)
    np.testing.assert_array_equal(S, S0)


def _span_maps(q, k, v, g, beta, bounds, form):
    """Per span: F (the state from the identity with v = 0) and E (the state
    from zero), both by a forward form of the oracle."""
    dk = q.shape[1]
    Fs, Es = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        zero_v = np.zeros((b - a, dk), np.float32)
        _, F = form(q[a:b], k[a:b], zero_v, g[a:b], beta[a:b], np.eye(dk))
        _, E = form(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], None)
        Fs.append(F)
        Es.append(E)
    return np.array(Fs), np.array(Es)


@pytest.mark.parametrize("form", sorted(FORMS))
def test_affine_scan_joins_spans(form):
    """The recurrence is affine in the state: scanning each span's map
    (F, E) from S0 reproduces the sequential state at every span boundary,
    and the last one is the final state (composition of span maps)."""
    rng = np.random.default_rng(5)
    T, dk, dv = 70, 6, 5
    bounds = [0, 1, 17, 40, 70]
    q, k, v, g, beta, S0 = pins._rand(rng, T, dk, dv)
    g[::7] = -9.0                     # beyond the floor: clamped inside every form
    Fs, Es = _span_maps(q, k, v, g, beta, bounds, FORMS[form])
    S = ref.affine_scan(Fs, Es, S0)
    assert S.shape == (len(bounds), dk, dv)
    for j, t in enumerate(bounds):
        _, S_ref = ref.seq(q[:t], k[:t], v[:t], g[:t], beta[:t], S0)
        assert np.abs(S[j] - S_ref).max() <= 1e-12 * max(1.0, np.abs(S_ref).max()), (form, j)


def test_affine_scan_special_cases():
    """Identity transitions sum the end states; zero transitions forget; an
    empty scan returns S0; a planted transposition of F is caught."""
    rng = np.random.default_rng(6)
    P, dk, dv = 3, 4, 3
    E = rng.normal(size=(P, dk, dv))
    S0 = rng.normal(size=(dk, dv))
    I = np.broadcast_to(np.eye(dk), (P, dk, dk))
    S = ref.affine_scan(I, E, S0)
    assert np.allclose(S[-1], S0 + E.sum(0), rtol=0, atol=1e-12)
    S = ref.affine_scan(np.zeros((P, dk, dk)), E, S0)
    assert np.allclose(S[-1], E[-1], rtol=0, atol=0)
    assert np.array_equal(ref.affine_scan(np.zeros((0, dk, dk)), np.zeros((0, dk, dv)), S0)[0], S0)
    F = rng.normal(size=(P, dk, dk))
    good = ref.affine_scan(F, E, S0)
    bad = ref.affine_scan(np.swapaxes(F, -1, -2), E, S0)
    assert np.abs(good - bad).max() > 1e-3
