"""The Python binding rejects every tensor that does not match the sizes the
C call will read or write, before any pointer reaches the library (CPU only:
each case fails in the binding's own checks, so nothing is launched).

The library derives every extent from q (or k) and v, so a shorter k, a bf16
S0, a CPU tensor or a wrong-sized output would otherwise be read or written
past its end on the device.
"""
import pytest
import torch

from linear_attention_recurrence_11_amd import binding

B, T, H, DK, DV = 2, 5, 3, 64, 32


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(binding.library_path()):
        from linear_attention_recurrence_11_amd import build
        build.build()
    return binding._load()


def fwd_inputs(dt=torch.bfloat16):
    z = lambda *s, d=dt: torch.zeros(s, dtype=d)
    return dict(q=z(B, T, H, DK), k=z(B, T, H, DK), v=z(B, T, H, DV), g=z(B, T, H, DK),
                beta=z(B, T, H), S0=z(B, H, DK, DV, d=torch.float32))


def call_fwd(ins, **kw):
    return binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"], **kw)


def expect(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


@pytest.mark.parametrize("name,bad,match", [
    ("k", lambda x: x[:, :4].contiguous(), "k has shape"),                 # shorter k
    ("g", lambda x: x[..., :32].contiguous(), "g has shape"),
    ("v", lambda x: x.float(), "v has dtype"),                             # fp32 v with bf16 q
    ("beta", lambda x: x[..., None].contiguous(), "beta has shape"),
    ("S0", lambda x: x.to(torch.bfloat16), "S0 has dtype"),                 # bf16 state
    ("S0", lambda x: x[:, :, :32].contiguous(), "S0 has shape"),
    ("k", lambda x: x.transpose(1, 2).contiguous().transpose(1, 2), "k must be contiguous"),
    ("q", lambda x: x[0], "q must have 4 dimensions"),
    ("k", lambda x: x.float().numpy(), "k must be a torch.Tensor"),
])
def test_forward_rejects_mismatched_inputs(name, bad, match):
    ins = fwd_inputs()
    ins[name] = bad(ins[name])
    exc = TypeError if "torch.Tensor" in match else ValueError
    expect(exc, match, call_fwd, ins)
    # the same checks guard the options entry point
    expect(exc, match, binding.kda_chunk_fwd_ex, ins["q"], ins["k"], ins["v"], ins["g"],
           ins["beta"], ins["S0"])


def test_forward_rejects_mismatched_outputs_and_buffers():
    ins = fwd_inputs()
    expect(ValueError, "o has shape", call_fwd, ins, o=torch.zeros(B, T, H, DV + 16))
    expect(ValueError, "o has dtype", call_fwd, ins, o=torch.zeros(B, T, H, DV, dtype=torch.float16))
    expect(ValueError, "S_T has dtype", call_fwd, ins,
           S_T=torch.zeros(B, H, DK, DV, dtype=torch.float64))
    expect(ValueError, "S_T has shape", call_fwd, ins, S_T=torch.zeros(B, H, DV, DK))
    expect(ValueError, "snapshots has shape", binding.kda_chunk_fwd_ex, ins["q"], ins["k"],
           ins["v"], ins["g"], ins["beta"], ins["S0"], snapshot_every=32,
           snapshots=torch.zeros(B, 1, H, DK, DV))
    expect(TypeError, "float32 or bfloat16", call_fwd, {n: x.double() for n, x in ins.items()})


def test_host_tensors_are_rejected():
    """Every shape and dtype right, but the tensors live in host memory."""
    ins = fwd_inputs()
    expect(ValueError, "q is on cpu", call_fwd, ins)
    meta = {n: x.to("meta") for n, x in ins.items()}
    expect(ValueError, "q is on meta", call_fwd, meta)


def test_stage_entry_points_check_their_tensors():
    ins = fwd_inputs()
    expect(ValueError, "beta has shape", binding.kda_chunk_prep, ins["q"], ins["k"], ins["g"],
           ins["beta"][:, :2].contiguous(), DV)
    ws = torch.zeros(16, dtype=torch.uint8)
    expect(ValueError, "S0 has dtype", binding.kda_chunk_state_pass, ins["v"], ws, DK,
           ins["S0"].half())
    expect(ValueError, "S0 has shape", binding.kda_chunk_state_pass, ins["v"], ws, DK + 64,
           ins["S0"])
    expect(ValueError, "workspace is required", binding.kda_chunk_state_pass, ins["v"], None, DK)
    expect(ValueError, "v is on cpu", binding.kda_chunk_state_pass, ins["v"], ws, DK, ins["S0"])


def dec_inputs(dt=torch.bfloat16, N=4):
    z = lambda *s, d=dt: torch.zeros(s, dtype=d)
    return dict(q=z(N, H, 128), k=z(N, H, 128), v=z(N, H, 64), g=z(N, H, 128), beta=z(N, H),
                S=z(N, H, 128, 64, d=torch.float32))


def test_decode_and_speculative_checks():
    d = dec_inputs()
    call = lambda **o: binding.kda_decode_step(*(o.get(n, d[n]) for n in ("q", "k", "v", "g", "beta",
                                                                          "S")))
    expect(ValueError, "S has dtype", call, S=d["S"].to(torch.bfloat16))
    expect(ValueError, "S has shape", call, S=d["S"][:2].contiguous())
    expect(ValueError, "v has shape", call, v=d["v"][:, :1].contiguous())
    expect(ValueError, "beta has dtype", call, beta=d["beta"].float())
    expect(ValueError, "S is required", call, S=None)
    expect(ValueError, "q is on cpu", call)
    expect(ValueError, "o has shape", binding.kda_decode_step_ex, d["q"], d["k"], d["v"], d["g"],
           d["beta"], d["S"], o=torch.zeros(4, H, 128))
    N, Td = 4, 3
    z = lambda *s, dd=torch.bfloat16: torch.zeros(s, dtype=dd)
    sp = dict(q=z(N, Td, H, 128), k=z(N, Td, H, 128), v=z(N, Td, H, 64), g=z(N, Td, H, 128),
              beta=z(N, Td, H))
    expect(ValueError, "g has shape", binding.kda_spec_verify, sp["q"], sp["k"], sp["v"],
           sp["g"][:, :2].contiguous(), sp["beta"], d["S"])
    expect(ValueError, "S has dtype", binding.kda_spec_verify, sp["q"], sp["k"], sp["v"], sp["g"],
           sp["beta"], d["S"].double())
    acc = torch.zeros(N, dtype=torch.int32)
    expect(ValueError, "accepted has dtype", binding.kda_spec_commit, sp["k"], sp["v"], sp["g"],
           sp["beta"], d["S"], acc.long())
    expect(ValueError, "accepted has shape", binding.kda_spec_commit, sp["k"], sp["v"], sp["g"],
           sp["beta"], d["S"], acc[:2].contiguous())
    expect(ValueError, "k is on cpu", binding.kda_spec_commit, sp["k"], sp["v"], sp["g"],
           sp["beta"], d["S"], acc)
    # the fused commit + next verify: the logged set takes its sizes from k1,
    # the drafts from q2 (a different token count), and both share N, H, dk, dv
    T2 = 2
    dr = dict(q=z(N, T2, H, 128), k=z(N, T2, H, 128), v=z(N, T2, H, 64), g=z(N, T2, H, 128),
              beta=z(N, T2, H))
    fused = lambda **o: binding.kda_spec_commit_verify(
        *(o.get(n, sp[n[:-1]]) for n in ("k1", "v1", "g1", "beta1")), o.get("acc", acc),
        *(o.get(n, dr[n[:-1]]) for n in ("q2", "k2", "v2", "g2", "beta2")), o.get("S", d["S"]),
        **({"o": o["o"]} if "o" in o else {}))
    expect(ValueError, "v1 has shape", fused, v1=sp["v"][:, :2].contiguous())
    expect(ValueError, "k2 has shape", fused, k2=sp["k"])
    expect(ValueError, "beta2 has dtype", fused, beta2=dr["beta"].float())
    expect(ValueError, "accepted has shape", fused, acc=acc[:3].contiguous())
    expect(ValueError, "S has dtype", fused, S=d["S"].to(torch.bfloat16))
    expect(ValueError, "o has shape", fused, o=torch.zeros(N, Td, H, 64))
    expect(ValueError, "k1 is on cpu", fused)
