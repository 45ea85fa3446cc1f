"""Pins for a per-(batch, head) KDA forward `fwd(q, k, v, g, beta, S0) -> (o, S_T)`.

Each pin checks the function against something other than itself: a closed
form, an invariant the recurrence fixes, a special case that reduces to a
simpler textbook recurrence, or an independently derived form. The recurrence
(decay rows of S by e^g with g floored at -5, delta-rule erase against the
decayed state with write strength beta, write k u^T, read o = S^T q after the
write) is the one on the pages: "K3 tech report" transcript (write strength,
channel-wise forgetting, the -5 log-decay floor, 16-token tiles);
"177: Kimi K3 in Detail" section 15 (delta rule, channel-wise forget gates,
lower bound on retention); "Kimi K3 goes trillion-scale ..." subtitles cue 14.

Inputs are float32 arrays (exactly representable for the C oracle); every pin
returns the largest relative deviation it found, and `PINS` lists
(name, function, tolerance).
"""
import numpy as np


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(rng, T, dk, dv, s0=True, gscale=1.0):
    f = np.float32
    q = _unit(rng.standard_normal((T, dk))).astype(f)
    k = _unit(rng.standard_normal((T, dk))).astype(f)
    v = rng.standard_normal((T, dv)).astype(f)
    g = (-gscale * np.log1p(np.exp(rng.standard_normal((T, dk))))).astype(f)
    beta = (1 / (1 + np.exp(-rng.standard_normal(T)))).astype(f)
    S0 = rng.standard_normal((dk, dv)).astype(f) * f(0.3) if s0 else None
    return q, k, v, g, beta, S0


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def pin_chunked(fwd, rng):
    """The independently derived chunk form (oracle.ref.chunked, chunk sizes
    16, 5 and 1, ragged last chunk) gives the same result as `fwd`."""
    from oracle import ref
    q, k, v, g, beta, S0 = _rand(rng, 37, 8, 5)
    o, S = fwd(q, k, v, g, beta, S0)
    worst = 0.0
    for C in (16, 5, 1):
        oc, Sc = ref.chunked(q, k, v, g, beta, S0, C=C)
        worst = max(worst, _rel(o, oc), _rel(S, Sc))
    return worst


def pin_beta_zero(fwd, rng):
    """beta = 0: nothing is written, S_t = Diag(exp(sum_{s<=t} g_s)) S0 and
    o_t = S_t^T q_t (the decay alone, applied per key channel = row)."""
    q, k, v, g, beta, S0 = _rand(rng, 20, 6, 4, gscale=0.5)
    beta = np.zeros_like(beta)
    o, S = fwd(q, k, v, g, beta, S0)
    cum = np.cumsum(np.clip(g.astype(np.float64), -5, 0), axis=0)
    o_ref = np.stack([(np.exp(cum[t])[:, None] * S0).T @ q[t] for t in range(20)])
    S_ref = np.exp(cum[-1])[:, None] * S0
    return max(_rel(o, o_ref), _rel(S, S_ref))


def pin_overwrite(fwd, rng):
    """beta = 1, g = 0, S0 = 0, orthonormal keys (some repeated): the delta rule
    overwrites, so S_T^T k_j returns the value last written under key k_j."""
    dk, dv = 8, 3
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:5].astype(np.float32)           # 5 orthonormal rows
    order = [0, 1, 2, 3, 4, 1, 3, 1]              # keys 1 and 3 rewritten
    T = len(order)
    k = keys[order]
    v = rng.standard_normal((T, dv)).astype(np.float32)
    q = k.copy()
    g = np.zeros((T, dk), np.float32)
    beta = np.ones(T, np.float32)
    o, S = fwd(q, k, v, g, beta, None)
    last = {}
    for t, j in enumerate(order):
        last[j] = v[t]
    # keys are orthonormal only to float32 rounding: allow ~1e-6
    got = np.stack([S.T @ keys[j].astype(np.float64) for j in sorted(last)])
    want = np.stack([last[j] for j in sorted(last)])
    return _rel(got, want)


def pin_self_read(fwd, rng):
    """beta_t = 1, ||k_t|| = 1, q_t = k_t: (I - k k^T) k = 0, so o_t = v_t for
    any decay and any prior state."""
    q, k, v, g, beta, S0 = _rand(rng, 25, 8, 5)
    k = _unit(k.astype(np.float64)).astype(np.float32)
    kk = k.astype(np.float64)
    # exact unit norm in float32 is not available; the identity holds to ~1e-7
    beta = np.ones_like(beta)
    o, S = fwd(k, k, v, g, beta, S0)
    norm_dev = float(np.abs((kk ** 2).sum(-1) - 1).max())
    return max(_rel(o, v) - 10 * norm_dev * float(np.abs(S0).max() + np.abs(v).max()), 0.0)


def pin_scalar_gate(fwd, rng):
    """Same log-decay on every channel: the recurrence reduces to the scalar-gated
    delta rule S_t = a_t (I - beta k k^T) S_{t-1} + beta k v^T with a = e^{g_t}
    (the decay commutes with the erase), written here independently."""
    q, k, v, g, beta, S0 = _rand(rng, 30, 6, 4)
    gs = g[:, :1].repeat(6, axis=1)
    o, S = fwd(q, k, v, gs, beta, S0)
    Sr = S0.astype(np.float64)
    orf = []
    for t in range(30):
        a = np.exp(max(min(float(gs[t, 0]), 0.0), -5.0))
        kt = k[t].astype(np.float64)
        Sr = a * (Sr - beta[t] * np.outer(kt, kt @ Sr)) + beta[t] * np.outer(kt, v[t])
        orf.append(Sr.T @ q[t])
    return max(_rel(o, np.array(orf)), _rel(S, Sr))


def pin_scalar_state(fwd, rng):
    """dk = dv = 1: s_t = (1 - beta_t k_t^2) e^{g_t} s_{t-1} + beta_t k_t v_t,
    o_t = q_t s_t (closed-form scalar recurrence)."""
    T = 40
    # |k| <= 1 and beta in [0, 1] keep |1 - beta k^2| <= 1 (no rounding blow-up)
    q = rng.standard_normal((T, 1)).astype(np.float32)
    k = rng.uniform(-1, 1, (T, 1)).astype(np.float32)
    v = rng.standard_normal((T, 1)).astype(np.float32)
    g = (-3 * rng.random((T, 1))).astype(np.float32)
    beta = rng.random(T).astype(np.float32)
    S0 = np.array([[0.7]], np.float32)
    o, S = fwd(q, k, v, g, beta, S0)
    s = float(S0[0, 0])
    orf = []
    for t in range(T):
        kt, bt = float(k[t, 0]), float(beta[t])
        s = (1 - bt * kt * kt) * np.exp(float(g[t, 0])) * s + bt * kt * float(v[t, 0])
        orf.append(float(q[t, 0]) * s)
    return max(_rel(np.ravel(o), orf), _rel(np.ravel(S), [s]))


def pin_linearity(fwd, rng):
    """For fixed q, k, g, beta the map (S0, V) -> (O, S_T) is linear:
    f(S0, V1 + V2) = f(S0, V1) + f(0, V2)."""
    q, k, v1, g, beta, S0 = _rand(rng, 24, 6, 4)
    # multiples of 1/64 of modest size: v1 + v2 is exact in float32
    v1 = (np.round(v1 * 64) / 64).astype(np.float32)
    v2 = (np.round(rng.standard_normal(v1.shape) * 64) / 64).astype(np.float32)
    v12 = (v1 + v2).astype(np.float32)
    oa, Sa = fwd(q, k, v12, g, beta, S0)
    ob, Sb = fwd(q, k, v1, g, beta, S0)
    oc, Sc = fwd(q, k, v2, g, beta, np.zeros_like(S0))
    return max(_rel(oa, ob + oc), _rel(Sa, Sb + Sc))


def pin_columns(fwd, rng):
    """Permuting the value columns of V and S0 permutes the columns of O and S_T
    the same way (columns of the state evolve independently)."""
    q, k, v, g, beta, S0 = _rand(rng, 21, 5, 6)
    perm = rng.permutation(6)
    o, S = fwd(q, k, v, g, beta, S0)
    op, Sp = fwd(q, k, np.ascontiguousarray(v[:, perm]), g, beta, np.ascontiguousarray(S0[:, perm]))
    return max(_rel(op, o[:, perm]), _rel(Sp, S[:, perm]))


def pin_split_resume(fwd, rng):
    """Running tokens [0, T) equals running [0, T1) then [T1, T) from its state."""
    q, k, v, g, beta, S0 = _rand(rng, 33, 6, 4)
    o, S = fwd(q, k, v, g, beta, S0)
    worst = 0.0
    for T1 in (1, 16, 20):
        o1, S1 = fwd(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], S0)
        o2, S2 = fwd(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], S1)
        worst = max(worst, _rel(np.concatenate([o1, o2]), o), _rel(S2, S))
    return worst


def pin_steps(fwd, rng):
    """Single-token steps chained through the state equal one call over all
    tokens (a decode step is the T = 1 case)."""
    q, k, v, g, beta, S0 = _rand(rng, 12, 5, 3)
    o, S = fwd(q, k, v, g, beta, S0)
    St, outs = S0, []
    for t in range(12):
        ot, St = fwd(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], St)
        outs.append(ot[0])
    return max(_rel(np.array(outs), o), _rel(St, S))


def pin_contractive(fwd, rng):
    """With unit keys, beta in [0,1] and g <= 0 each step obeys
    ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||_2 (I - beta k k^T and the decay
    have spectral norm <= 1). Returns the largest violation (0 when it holds)."""
    q, k, v, g, beta, S0 = _rand(rng, 30, 6, 4)
    k = _unit(k.astype(np.float64)).astype(np.float32)
    St = S0
    worst = 0.0
    for t in range(30):
        _, Sn = fwd(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], St)
        bound = np.linalg.norm(np.asarray(St, np.float64), 2) + beta[t] * np.linalg.norm(v[t])
        worst = max(worst, (np.linalg.norm(Sn, 2) - bound) / bound)
        St = Sn
    return max(worst - 1e-6, 0.0)


def pin_clamp(fwd, rng):
    """Log-decays outside [-5, 0] act as the nearest bound (the -5 floor)."""
    q, k, v, g, beta, S0 = _rand(rng, 18, 5, 3)
    g2 = g.copy()
    g2[::3] = -9.0
    g2[1::5] = 2.5
    g3 = np.clip(g2, -5, 0)
    o2, S2 = fwd(q, k, v, g2, beta, S0)
    o3, S3 = fwd(q, k, v, g3, beta, S0)
    return max(_rel(o2, o3), _rel(S2, S3))


def pin_highprec(fwd, rng):
    """Agreement with the recurrence evaluated at 50 significant digits."""
    from oracle import exact
    q, k, v, g, beta, S0 = _rand(rng, 9, 3, 2)
    o, S = fwd(q, k, v, g, beta, S0)
    om, Sm = exact.seq_mp(q.tolist(), k.tolist(), v.tolist(), g.tolist(), beta.tolist(), S0.tolist())
    return max(_rel(o, om), _rel(S, Sm))


PINS = [
    ("chunked", pin_chunked, 1e-12),
    ("beta_zero", pin_beta_zero, 1e-13),
    ("overwrite", pin_overwrite, 1e-5),
    ("self_read", pin_self_read, 1e-5),
    ("scalar_gate", pin_scalar_gate, 1e-12),
    ("scalar_state", pin_scalar_state, 1e-12),
    ("linearity", pin_linearity, 1e-12),
    ("columns", pin_columns, 1e-15),
    ("split_resume", pin_split_resume, 1e-13),
    ("steps", pin_steps, 1e-13),
    ("contractive", pin_contractive, 0.0),
    ("clamp", pin_clamp, 0.0),
    ("highprec", pin_highprec, 1e-13),
]


def run_all(fwd, seed=7):
    """{pin name: (deviation, tolerance, passed)} for every pin."""
    out = {}
    for name, fn, tol in PINS:
        rng = np.random.default_rng(seed)
        try:
            dev = fn(fwd, rng)
        except Exception as e:  # a shape mistake surfaces as an exception
            dev = float("inf")
            name = name + " (raised %s)" % type(e).__name__
        ok = bool(np.isfinite(dev) and dev <= tol)
        out[name] = (dev, tol, ok)
    return out
