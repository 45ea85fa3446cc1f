"""Bounds of the method on the GPU, through the C ABI, against the fp64 oracle.

- Log-decays outside [-5, 0] act as the bound: the decay floor of -5
  ("K3 tech report" podcast transcript, the exchange on the lower log-decay
  bound; "Kimi K3 goes trillion-scale with sparse MoE efficiency" subtitles,
  cue 14) and the cap at 0 (no growth). Every entry point clamps each g
  element before use; the oracle clamps too. Values -9, -5.5, +0.5 and +3
  are mixed into otherwise normal inputs, and the results must equal the
  oracle's within the bar and, bit for bit, the results for the pre-clamped
  log-decays.
- The sigmoid gate at large logits (the exponential overflows or underflows
  in fp32) gives the limits -5 and 0.
- Large values: v ~ N(0, (3e4)^2) and S0 ~ N(0, 1e6) with bf16 inputs, and a
  sequence whose values jump by twelve orders of magnitude and back, so the
  state and the per-chunk updates leave and re-enter the range of the
  matrix-core operand type.
"""
import numpy as np
import pytest
import torch

from gpucase import TOL, announce, gpu_forward, oracle_forward, rel_err
from linear_attention_recurrence_11_amd import binding, inputs
from oracle import c_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUT_OF_RANGE = (-9.0, -5.5, 0.5, 3.0)


def _plant(g, seed, frac=0.3):
    """g with a random `frac` of its entries replaced by out-of-range values
    (and its pre-clamped twin)."""
    gen = torch.Generator(device=g.device)
    gen.manual_seed(seed)
    pick = torch.rand(g.shape, generator=gen, device=g.device) < frac
    which = torch.randint(0, len(OUT_OF_RANGE), g.shape, generator=gen, device=g.device)
    vals = torch.tensor(OUT_OF_RANGE, device=g.device)[which].to(g.dtype)
    out = torch.where(pick, vals, g)
    return out, out.float().clamp(-5.0, 0.0).to(g.dtype)


def _oracle(ins, gate=0):
    to = inputs.to_oracle
    S0 = None if ins["S0"] is None else ins["S0"].detach().cpu().numpy()
    return c_oracle.fwd(to(ins["q"]), to(ins["k"]), to(ins["v"]), to(ins["g"]), to(ins["beta"]),
                        S0, gate=gate)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("dk", [64, 128])
def test_forward_clamps_out_of_range_log_decays(dt, dk):
    B, T, H, dv = 2, 333, 3, 64
    announce("forward out-of-range g", dt, "dk", dk)
    ins = inputs.make_forward(B, T, H, dk, dv, dt, "normal", seed=71 + dk, device=DEV)
    ins["g"], g_clamped = _plant(ins["g"], seed=72 + dk)
    assert float(ins["g"].float().min()) == -9.0 and float(ins["g"].float().max()) == 3.0
    o, ST = gpu_forward(ins)
    o_ref, S_ref = oracle_forward(ins)
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(ST.cpu().numpy(), S_ref)
    announce("  err_o=%.3g err_S=%.3g" % (eo, es))
    assert eo <= TOL[dt] and es <= TOL[dt]
    assert bool(torch.isfinite(o).all())
    o2, ST2 = gpu_forward(dict(ins, g=g_clamped))
    assert torch.equal(o, o2) and torch.equal(ST, ST2)


def test_forward_all_tokens_beyond_the_floor():
    """Every log-decay far below the floor: each chunk's reciprocal scaling is
    exactly e^80 at its largest, the bound the 16-token tile is built on."""
    ins = inputs.make_forward(1, 200, 2, 128, 128, "bf16", "normal", seed=73, device=DEV)
    ins["g"] = torch.full_like(ins["g"], -40.0)
    announce("forward g = -40 everywhere")
    o, ST = gpu_forward(ins)
    o_ref, S_ref = oracle_forward(ins)
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(ST.cpu().numpy(), S_ref)
    announce("  err_o=%.3g err_S=%.3g" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_clamps_out_of_range_log_decays(dt):
    N, steps, H, dk, dv = 9, 4, 3, 128, 128
    announce("decode out-of-range g", dt)
    d = inputs.make_decode(N, steps, H, dk, dv, dt, seed=74, device=DEV)
    d["g"], g_clamped = _plant(d["g"], seed=75)
    S, S2 = d["S"].clone(), d["S"].clone()
    outs, outs2 = [], []
    for s in range(steps):
        outs.append(binding.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s],
                                            d["beta"][s], S))
        outs2.append(binding.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], g_clamped[s],
                                             d["beta"][s], S2))
    torch.cuda.synchronize()
    seq = {n: d[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "beta")}
    seq["S0"] = d["S"]
    o_ref, S_ref = _oracle(seq)
    o = torch.stack(outs, 1)
    assert rel_err(o.cpu().numpy(), o_ref) <= 1e-4
    assert rel_err(S.cpu().numpy(), S_ref) <= 1e-4
    assert torch.equal(o, torch.stack(outs2, 1)) and torch.equal(S, S2)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_spec_verify_and_commit_clamp_out_of_range_log_decays(dt):
    N, T, H, dk, dv = 5, 6, 2, 128, 64
    announce("spec out-of-range g", dt)
    ins = inputs.make_forward(N, T, H, dk, dv, dt, "normal", seed=76, device=DEV)
    ins["g"], g_clamped = _plant(ins["g"], seed=77)
    o = binding.kda_spec_verify(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"])
    o2 = binding.kda_spec_verify(ins["q"], ins["k"], ins["v"], g_clamped, ins["beta"], ins["S0"])
    S = ins["S0"].clone()
    binding.kda_spec_commit(ins["k"], ins["v"], ins["g"], ins["beta"], S,
                            torch.full((N,), T, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(ins)
    assert rel_err(o.cpu().numpy(), o_ref) <= 1e-4
    assert rel_err(S.cpu().numpy(), S_ref) <= 1e-4
    assert torch.equal(o, o2)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_sigmoid_gate_at_large_logits(dt):
    """Logits whose exponential overflows or underflows fp32 (|x| >= 100)
    and moderate ones, against the oracle's gate."""
    ins = inputs.make_forward(2, 150, 2, 128, 64, dt, "normal", seed=78, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(79)
    choice = torch.tensor([-1e4, -200.0, -100.0, -30.0, -3.0, 0.0, 3.0, 30.0, 100.0, 200.0, 1e4],
                          device=DEV)
    ins["g"] = choice[torch.randint(0, len(choice), ins["g"].shape, generator=gen,
                                    device=DEV)].to(ins["g"].dtype)
    announce("sigmoid gate, large logits", dt)
    o, ST, _ = binding.kda_chunk_fwd_ex(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"],
                                        ins["S0"], gate=binding.KDA_GATE_SIGMOID)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(ins, gate=c_oracle.GATE_SIGMOID)
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(ST.cpu().numpy(), S_ref)
    announce("  err_o=%.3g err_S=%.3g" % (eo, es))
    assert eo <= TOL[dt] and es <= TOL[dt]
    # token 0 of each sequence as one decode step of B requests
    t0 = {n: ins[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta")}
    S = ins["S0"].clone()
    od = binding.kda_decode_step_ex(t0["q"], t0["k"], t0["v"], t0["g"], t0["beta"], S,
                                    gate=binding.KDA_GATE_SIGMOID)
    torch.cuda.synchronize()
    one = {n: ins[n][:, :1].contiguous() for n in ("q", "k", "v", "g", "beta")}
    one["S0"] = ins["S0"]
    o1_ref, S1_ref = _oracle(one, gate=c_oracle.GATE_SIGMOID)
    assert rel_err(od.cpu().numpy(), o1_ref[:, 0]) <= 1e-4
    assert rel_err(S.cpu().numpy(), S1_ref) <= 1e-4


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 48)])
def test_large_values_bf16(dk, dv):
    """v ~ N(0, (3e4)^2), S0 ~ N(0, 1e6): entries of v, of the state and of the
    updates far above the fp16 maximum (65504)."""
    B, T, H = 2, 500, 3
    announce("large values", dk, dv)
    ins = inputs.make_forward(B, T, H, dk, dv, "bf16", "normal", seed=80 + dk + dv, device=DEV)
    ins["v"] = (ins["v"].float() * 3e4).to(torch.bfloat16)
    ins["S0"] = ins["S0"] * (1e3 / 0.02)
    assert float(ins["v"].float().abs().max()) > 65504
    o, ST = gpu_forward(ins)
    o_ref, S_ref = oracle_forward(ins)
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(ST.cpu().numpy(), S_ref)
    announce("  err_o=%.3g err_S=%.3g" % (eo, es))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # the output dtype option and snapshots carry the same values
    ob, _, sn = binding.kda_chunk_fwd_ex(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"],
                                         ins["S0"], out_dtype=torch.bfloat16, snapshot_every=64)
    torch.cuda.synchronize()
    assert torch.equal(ob, o.to(torch.bfloat16))
    _, S_pre = oracle_forward({n: (x[:, :256] if n != "S0" else x) for n, x in ins.items()})
    assert rel_err(sn[:, 3].cpu().numpy(), S_pre) <= TOL["bf16"]


@pytest.mark.parametrize("B", [4, 8], ids=["2_slices", "4_slices"])
def test_large_values_in_multi_slice_workgroups(B):
    """Large values where the plain pass serves 2 or 4 slices per workgroup
    (512 and 1024 slices of 128 x 128 heads): slices whose fp16 operands
    overflow there raise their range flag, and the scaled pass (one slice per
    workgroup) redoes them. Only the even heads get the large v, so flagged
    and unflagged slices mix."""
    T, H, dk, dv = 96, 16, 128, 128
    announce("large values, multi-slice workgroups, B", B)
    ins = inputs.make_forward(B, T, H, dk, dv, "bf16", "normal", seed=84 + B, device=DEV)
    v = ins["v"].float()
    v[:, :, ::2] *= 3e4   # even heads
    ins["v"] = v.to(torch.bfloat16)
    ins["S0"] = ins["S0"] * (1e3 / 0.02)
    o, ST = gpu_forward(ins)
    o_ref, S_ref = oracle_forward(ins)
    for hs in (slice(0, None, 2), slice(1, None, 2)):   # each group of heads on its own scale
        eo = rel_err(o[:, :, hs].cpu().numpy(), o_ref[:, :, hs])
        es = rel_err(ST[:, hs].cpu().numpy(), S_ref[:, hs])
        announce("  heads %s: err_o=%.3g err_S=%.3g" % (hs, eo, es))
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_values_jump_by_twelve_orders_and_back():
    """A burst of values near 1e12 in the middle of a sequence, then 64 tokens
    at the -5 floor that forget it, then ordinary values again: the outputs
    after the burst is forgotten must keep their own relative precision."""
    B, T, H, dk, dv = 1, 1024, 2, 128, 64
    ins = inputs.make_forward(B, T, H, dk, dv, "bf16", "normal", seed=83, device=DEV)
    t0, t1 = 320, 352
    v = ins["v"].float()
    v[:, t0:t1] *= 1e12
    ins["v"] = v.to(torch.bfloat16)
    g = ins["g"].float()
    g[:, t1:t1 + 64] = -5.0
    ins["g"] = g.to(torch.bfloat16)
    announce("value burst")
    o, ST = gpu_forward(ins)
    o_ref, S_ref = oracle_forward(ins)
    oh = o.cpu().numpy()
    e_all = rel_err(oh, o_ref)
    e_burst = rel_err(oh[:, t0:t1], o_ref[:, t0:t1])
    e_after = rel_err(oh[:, t1 + 96:], o_ref[:, t1 + 96:])
    e_before = rel_err(oh[:, :t0], o_ref[:, :t0])
    es = rel_err(ST.cpu().numpy(), S_ref)
    announce("  err all=%.3g before=%.3g burst=%.3g after=%.3g S=%.3g"
             % (e_all, e_before, e_burst, e_after, es))
    assert max(e_all, e_before, e_burst, e_after, es) <= TOL["bf16"]
    assert np.abs(o_ref[:, t1 + 96:]).max() < 1e3     # the burst really was forgotten
