"""NumPy fp64 forms of the KDA recurrence (test infrastructure only).

seq      the per-token sequential definition, step by step:
           g <- clamp(g, -5, 0); P = Diag(e^g) S; u = beta (v - P^T k);
           S = P + k u^T; o = S^T q.
         Decay floor of -5: "K3 tech report" transcript (the exchange on the
         lower log-decay bound) and "Kimi K3 goes trillion-scale ..." subtitles,
         cue 14. Delta rule with channel-wise forget gate and a fixed-size state:
         "177: Kimi K3 in Detail", section 15; same subtitles, cue 14.

chunked  the same result reached chunk by chunk, written out matrix by matrix
         from the chunk form obtained by unrolling the recurrence over a chunk
         of C tokens (the 16-token tile of the "K3 tech report" transcript):
           Gamma_r = sum_{s<=r} g_s (per key channel), gamma = Gamma_C
           Qt = e^Gamma * Q, Kt = e^Gamma * K, Kh = e^-Gamma * K, Kb = e^(gamma-Gamma) * K
           A = strictly_lower(diag(beta) Kt Kh^T),  M = lower_incl(Qt Kh^T)
           Tm = (I + A)^-1,  W = Tm diag(beta) Kt,  Ut = Tm diag(beta) V
           U = Ut - W S0,  O = Qt S0 + M U,  S_C = Diag(e^gamma) S0 + Kb^T U
         A last chunk shorter than C is just a shorter chunk.

chunk_terms
         one chunk's matrices of that form (used by chunked, and by tests of
         the prepared per-chunk operands).

affine_scan
         the states entering consecutive spans of a sequence from each span's
         affine map S_out = F S_in + E (F: the span's state transition, the
         state it reaches from the identity with v = 0; E: the state it
         reaches from zero): S[0] = S0, S[r+1] = F[r] S[r] + E[r]. The
         recurrence is affine in the state, which is what lets a sequence be
         split over devices and joined afterwards (KDA context parallelism:
         "K3 tech report" transcript, the exchange on recreating the training
         efficiency; "Kimi K3 goes trillion-scale ..." subtitles, cue 22).

Arrays are per (batch, head): q, k, g [T, dk]; v [T, dv]; beta [T]; S0 [dk, dv].
All arithmetic is float64.
"""
import numpy as np


def clamp_decay(g):
    """Clamp log-decay to [-5, 0]; NaN stays NaN (np.clip propagates NaN)."""
    return np.clip(np.asarray(g, np.float64), -5.0, 0.0)


def seq(q, k, v, g, beta, S0=None):
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    g = clamp_decay(g)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.empty((T, dv))
    for t in range(T):
        P = np.exp(g[t])[:, None] * S
        u = beta[t] * (v[t] - P.T @ k[t])
        S = P + np.outer(k[t], u)
        o[t] = S.T @ q[t]
    return o, S


def chunk_terms(q, k, g, beta):
    """The chunk form's per-chunk matrices for one chunk of n tokens (q, k, g
    [n, dk], beta [n]; g already clamped): Gam, gam, Qt, Kt, Kh, Kb, A, M,
    Tm, W and Tb = Tm diag(beta), in the notation of the module docstring."""
    n = q.shape[0]
    Gam = np.cumsum(g, axis=0)
    gam = Gam[-1]
    Qt = np.exp(Gam) * q
    Kt = np.exp(Gam) * k
    Kh = np.exp(-Gam) * k
    Kb = np.exp(gam[None, :] - Gam) * k
    A = np.tril(beta[:, None] * (Kt @ Kh.T), -1)
    M = np.tril(Qt @ Kh.T)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ (beta[:, None] * Kt)
    return dict(Gam=Gam, gam=gam, Qt=Qt, Kt=Kt, Kh=Kh, Kb=Kb, A=A, M=M, Tm=Tm, W=W,
                Tb=Tm * beta[None, :])


def chunked(q, k, v, g, beta, S0=None, C=16):
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    g = clamp_decay(g)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.empty((T, dv))
    for start in range(0, T, C):
        sl = slice(start, min(start + C, T))
        c = chunk_terms(q[sl], k[sl], g[sl], beta[sl])
        Ut = c["Tb"] @ v[sl]
        U = Ut - c["W"] @ S
        o[sl] = c["Qt"] @ S + c["M"] @ U
        S = np.exp(c["gam"])[:, None] * S + c["Kb"].T @ U
    return o, S


def seq_batched(q, k, v, g, beta, S0=None, fn=seq, **kw):
    """Apply a per-(b,h) form to [B,T,H,d]-laid-out arrays."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv))
    ST = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            s0 = None if S0 is None else S0[b, h]
            o[b, :, h], ST[b, h] = fn(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h],
                                      beta[b, :, h], s0, **kw)
    return o, ST


def affine_scan(F, E, S0=None):
    """F [P, ..., dk, dk], E [P, ..., dk, dv], S0 [..., dk, dv] or None ->
    S [P + 1, ..., dk, dv] with S[0] = S0 and S[r+1] = F[r] @ S[r] + E[r]."""
    F, E = np.asarray(F, np.float64), np.asarray(E, np.float64)
    S = np.empty((F.shape[0] + 1,) + E.shape[1:])
    S[0] = 0.0 if S0 is None else np.asarray(S0, np.float64)
    for r in range(F.shape[0]):
        S[r + 1] = F[r] @ S[r] + E[r]
    return S
