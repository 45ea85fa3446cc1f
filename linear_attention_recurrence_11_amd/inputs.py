"""Seeded synthetic inputs for the KDA workloads.

This module holds only random draws and the input distributions of the
workloads (normalisation of q and k, the sigmoid of the write strength, the
softplus of the log-decay); none of the recurrence's arithmetic. Both the HIP
path and the fp64 oracle receive the tensors it returns.

Recipe (per workload, one torch generator seeded with the workload seed):
  draw order q, k, v, beta, g, S0, then the pinned-channel mask, then (decode)
  the per-step tensors. Every normal draw is fp32, made in blocks of at most
  65536 tokens along T, transformed in fp32, then rounded to the input dtype
  (round-to-nearest-even for bf16).
    q, k  ~ N(0,1), divided by max(||x||_2, 1e-6) over the key dimension
    v     ~ N(0,1)
    beta  = sigmoid(N(0,1))
    g     = max(-5, -softplus(N(0,1))) per channel; with a pinned fraction p,
            a seeded random p*dk channels of every head are -5 at every token
    S0    = 0, or 0.02 * N(0,1) in fp32
    gate logits (for the sigmoid-gate option, replacing g): 2 * N(0,1) - 2,
            so the log-decay -5 sigmoid(x) averages about -1 with a spread
            over most of (-5, 0)
Layouts: q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; S0 [B,H,dk,dv].
Decode steps: q, k, g [steps,N,H,dk]; v [steps,N,H,dv]; beta [steps,N,H];
state S [N,H,dk,dv] fp32.
"""
import torch

BLOCK = 65536


def _dt(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _blocked(gen, B, T, H, d, device, transform, dtype):
    """Draw [B,T,H,d] (or [B,T,H] when d is None) in T-blocks, transform in fp32."""
    shape_tail = (H,) if d is None else (H, d)
    out = torch.empty((B, T) + shape_tail, dtype=dtype, device=device)
    for t0 in range(0, T, BLOCK):
        t1 = min(T, t0 + BLOCK)
        x = _normal(gen, (B, t1 - t0) + shape_tail, device)
        out[:, t0:t1] = transform(x).to(dtype)
    return out


def _unit(x):
    return x / torch.clamp(torch.linalg.vector_norm(x, dim=-1, keepdim=True), min=1e-6)


def _decay(x):
    return torch.clamp(-torch.nn.functional.softplus(x), min=-5.0)


def _logit(x):
    return 2.0 * x - 2.0


def make_generator(seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def make_forward(B, T, H, dk, dv, in_dtype="bf16", s0="zero", pinned_fraction=0.0,
                 seed=0, device="cpu", gate_logits=False):
    """Forward inputs; with gate_logits=True, g holds gate logits (recipe above)
    instead of log-decays."""
    dt = _dt(in_dtype)
    gen = make_generator(seed, device)
    q = _blocked(gen, B, T, H, dk, device, _unit, dt)
    k = _blocked(gen, B, T, H, dk, device, _unit, dt)
    v = _blocked(gen, B, T, H, dv, device, lambda x: x, dt)
    beta = _blocked(gen, B, T, H, None, device, torch.sigmoid, dt)
    g = _blocked(gen, B, T, H, dk, device, _logit if gate_logits else _decay, dt)
    if s0 == "zero":
        S0 = None
    else:
        S0 = 0.02 * _normal(gen, (B, H, dk, dv), device)
    if pinned_fraction > 0:
        npin = int(round(pinned_fraction * dk))
        keys = torch.rand((B, H, dk), generator=gen, device=device)
        idx = torch.argsort(keys, dim=-1)[..., :npin]
        mask = torch.zeros((B, H, dk), dtype=torch.bool, device=device)
        mask.scatter_(-1, idx, True)
        for t0 in range(0, T, BLOCK):
            t1 = min(T, t0 + BLOCK)
            blk = g[:, t0:t1]
            blk.masked_fill_(mask[:, None], -5.0)
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)


def make_decode(N, steps, H, dk, dv, in_dtype="bf16", seed=0, device="cpu", gate_logits=False):
    dt = _dt(in_dtype)
    gen = make_generator(seed, device)
    S = 0.02 * _normal(gen, (N, H, dk, dv), device)
    q = _unit(_normal(gen, (steps, N, H, dk), device)).to(dt)
    k = _unit(_normal(gen, (steps, N, H, dk), device)).to(dt)
    v = _normal(gen, (steps, N, H, dv), device).to(dt)
    beta = torch.sigmoid(_normal(gen, (steps, N, H), device)).to(dt)
    g = (_logit if gate_logits else _decay)(_normal(gen, (steps, N, H, dk), device)).to(dt)
    return dict(S=S, q=q, k=k, v=v, g=g, beta=beta)


def make_workload(w, device="cpu", T=None, B=None):
    """Inputs for a configs.Workload (T or B may be overridden for sampled runs)."""
    if w.kind == "decode":
        return make_decode(B or w.B, T or w.T, w.H, w.dk, w.dv, w.in_dtype, w.seed, device)
    return make_forward(B or w.B, T or w.T, w.H, w.dk, w.dv, w.in_dtype, w.s0, w.pinned_fraction,
                        w.seed, device)


def to_oracle(x):
    """Tensor -> NumPy array the oracle accepts: float32 stays float32, bfloat16
    becomes its raw 16-bit pattern (uint16), float32 state stays float32."""
    x = x.detach().contiguous().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError("unsupported dtype %s" % x.dtype)
