"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding and the fp64 oracle on the same seeded inputs, and measure
max |x - ref| / rms(ref)."""
import os
import sys

import numpy as np
import torch

from linear_attention_recurrence_11_amd import binding, inputs
from oracle import c_oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.abs(x - ref).max() / rms) if rms > 0 else float(np.abs(x - ref).max())
    log = os.environ.get("KDA_ERR_LOG")
    if log:  # one line per comparison: test id, error
        with open(log, "a") as f:
            f.write("%s %.3e\n" % (os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], err))
    return err


def gpu_forward(ins, out_dtype=torch.float32, S_T=None, workspace=None):
    o, ST = binding.kda_chunk_fwd(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["S0"],
                                  out_dtype=out_dtype, S_T=S_T, workspace=workspace)
    torch.cuda.synchronize()
    return o, ST


def oracle_forward(ins):
    to = inputs.to_oracle
    S0 = None if ins["S0"] is None else ins["S0"].detach().cpu().numpy()
    return c_oracle.fwd(to(ins["q"]), to(ins["k"]), to(ins["v"]), to(ins["g"]), to(ins["beta"]), S0)


def head_slice(x, b, h):
    """[B,T,H,...] device tensor -> host NumPy oracle array [1,T,1,...] for (b,h)."""
    return inputs.to_oracle(x[b:b + 1, :, h:h + 1].contiguous())


def oracle_columns(ins, b, h, cols):
    """Oracle for value columns `cols` of head (b,h) over the full sequence."""
    q, k, v, g, beta = (head_slice(ins[n], b, h) for n in ("q", "k", "v", "g", "beta"))
    S0c = None
    if ins["S0"] is not None:
        S0c = ins["S0"][b, h][:, cols].detach().cpu().numpy()
    return c_oracle.fwd_cols(q, k, v, g, beta, 0, 0, cols, S0c)
