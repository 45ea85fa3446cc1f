"""kda_chunk_fwd_noalloc (the forward on the library's built-in scratch)
against kda_chunk_fwd on the same inputs, through the C ABI: two calls in a
row, the second smaller, each bit-identical to the workspace forward (same
kernels, same arithmetic) and within the oracle's bar."""
import pytest
import torch

from gpucase import TOL, announce, oracle_forward, rel_err
from linear_attention_recurrence_11_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(ins, out_dtype=torch.float32):
    B, T, H, _ = ins["q"].shape
    dk, dv = ins["q"].shape[-1], ins["v"].shape[-1]
    o_ref, S_ref = binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"],
                                         ins["S0"], out_dtype=out_dtype)
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device=DEV)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=DEV)
    binding.kda_chunk_fwd_noalloc(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"],
                                  o, S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_forward_twice(dt):
    # first call: large (near the scratch limit for bf16), then a smaller one
    big = (1, 2048, 32, 128, 128) if dt == "bf16" else (1, 1024, 16, 128, 128)
    small = (2, 77, 3, 64, 48)
    for shape, seed in ((big, 11), (small, 12)):
        announce("noalloc", dt, shape)
        ins = inputs.make_forward(*shape, dt, "normal", seed=seed, device=DEV)
        o, S, o_ref, S_ref = _both(ins)
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), shape
        o_or, S_or = oracle_forward(ins)
        eo, es = rel_err(o.cpu().numpy(), o_or), rel_err(S.cpu().numpy(), S_or)
        announce("  err_o=%.3g err_S=%.3g" % (eo, es))
        assert eo <= TOL[dt] and es <= TOL[dt]


def test_noalloc_large_values_and_in_place_state():
    """The rescaling pass (its flags live in the scratch too) and S_T = S0."""
    ins = inputs.make_forward(2, 300, 3, 128, 128, "bf16", "normal", seed=13, device=DEV)
    ins["v"] = (ins["v"].float() * 3e4).to(torch.bfloat16)
    ins["S0"] = ins["S0"] * 5e4
    o, S, o_ref, S_ref = _both(ins)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    S_in = ins["S0"].clone()
    o2 = torch.empty_like(o)
    binding.kda_chunk_fwd_noalloc(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], S_in, o2,
                                  S_in)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(S_in, S_ref)


def test_noalloc_rejects_work_beyond_the_scratch():
    ins = inputs.make_forward(1, 4096, 32, 128, 128, "bf16", "zero", seed=14, device=DEV)
    o = torch.empty((1, 4096, 32, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.KDAError) as exc:
        binding.kda_chunk_fwd_noalloc(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], None, o)
    assert exc.value.status == 8
