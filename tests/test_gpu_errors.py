"""Error paths through the Python binding on the GPU: an injected launch
failure surfaces as KDAError(KDA_ERR_HIP) with the outputs untouched, and
the next call runs normally; argument errors leave outputs untouched too."""
import pytest
import torch

from gpucase import announce
from linear_attention_recurrence_11_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_injected_failure_then_normal_call():
    ins = inputs.make_forward(1, 70, 2, 128, 64, "bf16", "normal", seed=5, device=DEV)
    announce("injected launch failure")
    o = torch.full((1, 70, 2, 64), 7.0, device=DEV)
    S = torch.full((1, 2, 128, 64), 7.0, device=DEV)
    binding.kda_debug_inject_launch_failures(1)
    try:
        with pytest.raises(binding.KDAError) as exc:
            binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"],
                                  o=o, S_T=S)
    finally:
        binding.kda_debug_inject_launch_failures(0)
    assert exc.value.status == 6
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((S == 7.0).all())
    o2, S2 = binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"],
                                   o=o, S_T=S)
    ref_o, ref_S = binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"],
                                         ins["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o) and torch.equal(S2, ref_S)


def test_rejected_arguments_leave_outputs_untouched():
    d = inputs.make_decode(3, 1, 2, 128, 128, "bf16", seed=6, device=DEV)
    S = d["S"].clone()
    o = torch.full((3, 2, 128), 7.0, device=DEV)
    with pytest.raises(binding.KDAError) as exc:   # unsupported head size, checked in C
        binding.kda_decode_step(d["q"][0][..., :96].contiguous(), d["k"][0][..., :96].contiguous(),
                                d["v"][0], d["g"][0][..., :96].contiguous(), d["beta"][0],
                                torch.zeros((3, 2, 96, 128), device=DEV), o=o)
    assert exc.value.status == 3
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and torch.equal(S, d["S"])
