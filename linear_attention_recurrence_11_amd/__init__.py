"""Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libkda.so (hand-written HIP kernels);
`binding` marshals torch tensors into it. Importing this package loads nothing;
the library is opened on first use and its absence is an error.
"""
from .binding import (KDAError, kda_abi_version, kda_chunk_fwd,  # noqa: F401
                      kda_chunk_fwd_workspace_size, kda_chunk_prep, kda_chunk_state_pass,
                      kda_decode_step, kda_status_str, library_path)
