"""The five synthetic KDA workloads, by shape and input recipe.

Each workload fixes shapes, dtypes and the distributions its inputs are drawn
from; `inputs.make_forward` / `inputs.make_decode` turn a workload and a seed
into tensors. Lengths follow the pages' context schedule: 64K tokens is a
pre-training length and 1M tokens the cool-down context ("K3 tech report"
transcript, the exchange on context extension).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "forward" or "decode"
    B: int               # batch (forward) / requests N (decode)
    T: int               # tokens per sequence (forward) / decode steps (decode)
    H: int
    dk: int
    dv: int
    in_dtype: str        # "f32" or "bf16"
    s0: str              # "zero" or "normal" (std 0.02, fp32)
    pinned_fraction: float = 0.0  # share of g channels per head held at -5
    seed: int = 0

    @property
    def tokens(self):
        return self.B * self.T


WORKLOADS = [
    Workload("fwd_f32_b1_h2_t256_d64", "forward", 1, 256, 2, 64, 64, "f32", "zero", seed=1234),
    Workload("fwd_bf16_b4_h16_t4096_d128", "forward", 4, 4096, 16, 128, 128, "bf16", "normal", seed=1235),
    Workload("prefill_bf16_b1_h32_t65536_d128", "forward", 1, 65536, 32, 128, 128, "bf16", "zero", seed=1236),
    Workload("prefill_bf16_b1_h32_t1048576_d128_pinned", "forward", 1, 1048576, 32, 128, 128, "bf16",
             "zero", pinned_fraction=0.5, seed=1237),
    Workload("decode_bf16_n256_h32_d128_64steps", "decode", 256, 64, 32, 128, 128, "bf16", "normal",
             seed=1238),
]
BY_NAME = {w.name: w for w in WORKLOADS}

SMALL_FWD = WORKLOADS[0]
MID_FWD = WORKLOADS[1]
PREFILL_64K = WORKLOADS[2]
PREFILL_1M = WORKLOADS[3]
DECODE = WORKLOADS[4]
