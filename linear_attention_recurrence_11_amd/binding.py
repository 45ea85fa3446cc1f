"""Thin Python binding of libkda.so (ctypes), same names as the C ABI.

Argument marshalling only: torch tensors supply device memory and the current
stream, every step of the computation runs in the library's HIP kernels. The
library is loaded from this package directory on first use; if it is missing
the call raises (there is no fallback path).
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# The argument lists below follow this version of include/kda.h.
ABI_VERSION = 2
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_LOG_DECAY, KDA_GATE_SIGMOID = 0, 1
_STATUS_OK = 0


class KDAError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, _status_text(status), status))


def library_path():
    return os.path.join(_PKG, "libkda.so")


def _load():
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise FileNotFoundError(
                "libkda.so is not built at %s; run `python -m linear_attention_recurrence_11_amd.build`"
                % path)
        lib = ctypes.CDLL(path)
        vp, i64, i, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        lib.kda_abi_version.restype = i
        lib.kda_abi_version.argtypes = []
        found = lib.kda_abi_version()
        if found != ABI_VERSION:
            raise RuntimeError("%s has ABI version %d, this binding expects %d; rebuild it"
                               % (path, found, ABI_VERSION))
        lib.kda_status_str.restype = ctypes.c_char_p
        lib.kda_status_str.argtypes = [i]
        lib.kda_chunk_fwd_workspace_size.restype = sz
        lib.kda_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i]
        lib.kda_chunk_fwd.restype = i
        lib.kda_chunk_fwd.argtypes = [vp] * 8 + [i64] * 5 + [i, i, vp, sz, vp]
        lib.kda_chunk_fwd_check.restype = i
        lib.kda_chunk_fwd_check.argtypes = [vp] * 8 + [i64] * 5 + [i, i, vp, sz]
        lib.kda_chunk_prep.restype = i
        lib.kda_chunk_prep.argtypes = [vp] * 4 + [i64] * 5 + [i, vp, sz, vp]
        lib.kda_chunk_state_pass.restype = i
        lib.kda_chunk_state_pass.argtypes = [vp, vp, sz, vp, vp, vp] + [i64] * 5 + [i, i, vp]
        lib.kda_decode_step.restype = i
        lib.kda_decode_step.argtypes = [vp] * 7 + [i64] * 4 + [i, i, vp]
        lib.kda_decode_step_check.restype = i
        lib.kda_decode_step_check.argtypes = [vp] * 7 + [i64] * 4 + [i, i]
        lib.kda_chunk_fwd_ex.restype = i
        lib.kda_chunk_fwd_ex.argtypes = [vp] * 8 + [i64] * 5 + [i, i, i, vp, i64, vp, sz, vp]
        lib.kda_chunk_fwd_ex_check.restype = i
        lib.kda_chunk_fwd_ex_check.argtypes = [vp] * 8 + [i64] * 5 + [i, i, i, vp, i64, vp, sz]
        lib.kda_decode_step_ex.restype = i
        lib.kda_decode_step_ex.argtypes = [vp] * 7 + [i64] * 4 + [i, i, i, vp]
        lib.kda_spec_verify.restype = i
        lib.kda_spec_verify.argtypes = [vp] * 7 + [i64] * 5 + [i, i, i, vp]
        lib.kda_spec_verify_check.restype = i
        lib.kda_spec_verify_check.argtypes = [vp] * 7 + [i64] * 5 + [i, i, i]
        lib.kda_spec_commit.restype = i
        lib.kda_spec_commit.argtypes = [vp] * 6 + [i64] * 5 + [i, i, vp]
        lib.kda_spec_commit_check.restype = i
        lib.kda_spec_commit_check.argtypes = [vp] * 6 + [i64] * 5 + [i, i]
        _LIB = lib
    return _LIB


def _status_text(status):
    try:
        return _load().kda_status_str(int(status)).decode()
    except Exception:
        return "status"


def _dcode(dtype):
    if dtype == torch.float32:
        return KDA_F32
    if dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError("KDA tensors must be float32 or bfloat16, got %s" % dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("KDA tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(0)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def kda_abi_version():
    return int(_load().kda_abi_version())


def kda_status_str(status):
    return _load().kda_status_str(int(status)).decode()


def kda_chunk_fwd_workspace_size(B, T, H, dk, dv, in_dtype):
    code = in_dtype if isinstance(in_dtype, int) else _dcode(in_dtype)
    return int(_load().kda_chunk_fwd_workspace_size(B, T, H, dk, dv, code))


def kda_chunk_fwd(q, k, v, g, beta, S0=None, *, o=None, S_T=None, out_dtype=torch.float32,
                  want_state=True, workspace=None, stream=None):
    """Chunkwise KDA forward. q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]
    (all float32 or all bfloat16, on one GPU); S0 [B,H,dk,dv] float32 or None.
    Returns (o [B,T,H,dv] out_dtype, S_T [B,H,dk,dv] float32 or None).
    Pass S_T=S0 to update the state in place."""
    lib = _load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dcode(q.dtype)
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    need = int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                           _ptr(S_T), B, T, H, dk, dv, code, _dcode(o.dtype), _ptr(workspace),
                           wbytes, _stream(stream, dev))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_chunk_fwd")
    return o, S_T


def kda_chunk_prep(q, k, g, beta, dv, *, workspace=None, stream=None):
    """First stage of kda_chunk_fwd: per-chunk operands into a workspace
    (allocated here when not given). Returns the workspace tensor."""
    lib = _load()
    B, T, H, dk = q.shape
    code = _dcode(q.dtype)
    need = int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_prep(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), B, T, H, dk, dv, code,
                            _ptr(workspace), wbytes, _stream(stream, q.device))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_chunk_prep")
    return workspace


def kda_chunk_state_pass(v, workspace, dk, S0=None, *, o=None, S_T=None, in_dtype=None,
                         out_dtype=torch.float32, want_state=True, stream=None):
    """Second stage of kda_chunk_fwd: the sequential pass from S0 over the chunks
    prepared in `workspace` (by kda_chunk_prep on the same sizes and in_dtype)."""
    lib = _load()
    B, T, H, dv = v.shape
    code = _dcode(v.dtype if in_dtype is None else in_dtype)
    dev = v.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_state_pass(_ptr(v), _ptr(workspace), wbytes, _ptr(S0), _ptr(o), _ptr(S_T),
                                  B, T, H, dk, dv, code, _dcode(o.dtype), _stream(stream, dev))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_chunk_state_pass")
    return o, S_T


def kda_decode_step(q, k, v, g, beta, S, *, o=None, out_dtype=torch.float32, stream=None):
    """One decode step for N requests. q, k, g [N,H,dk]; v [N,H,dv]; beta [N,H];
    S [N,H,dk,dv] float32, updated in place. Returns o [N,H,dv]."""
    lib = _load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=q.device)
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                             N, H, dk, dv, _dcode(q.dtype), _dcode(o.dtype),
                             _stream(stream, q.device))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_decode_step")
    return o


def kda_chunk_fwd_ex(q, k, v, g, beta, S0=None, *, gate=KDA_GATE_LOG_DECAY, snapshot_every=0,
                     snapshots=None, o=None, S_T=None, out_dtype=torch.float32, want_state=True,
                     workspace=None, stream=None):
    """kda_chunk_fwd with a gate option (KDA_GATE_SIGMOID: g holds gate logits)
    and state snapshots every `snapshot_every` tokens (0: none) into
    `snapshots` [B, T // snapshot_every, H, dk, dv] float32 (allocated here
    when not given). Returns (o, S_T, snapshots or None)."""
    lib = _load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dcode(q.dtype)
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    nsnap = T // snapshot_every if snapshot_every > 0 else 0
    if snapshots is None and nsnap > 0:
        snapshots = torch.empty((B, nsnap, H, dk, dv), dtype=torch.float32, device=dev)
    need = int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                              _ptr(S_T), B, T, H, dk, dv, code, _dcode(o.dtype), int(gate),
                              _ptr(snapshots), int(snapshot_every), _ptr(workspace), wbytes,
                              _stream(stream, dev))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_chunk_fwd_ex")
    return o, S_T, snapshots


def kda_decode_step_ex(q, k, v, g, beta, S, *, gate=KDA_GATE_LOG_DECAY, o=None,
                       out_dtype=torch.float32, stream=None):
    """kda_decode_step with a gate option. Returns o [N,H,dv]; S updated in place."""
    lib = _load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=q.device)
    st = lib.kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                                N, H, dk, dv, _dcode(q.dtype), _dcode(o.dtype), int(gate),
                                _stream(stream, q.device))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_decode_step_ex")
    return o


def kda_spec_verify(q, k, v, g, beta, S, *, gate=KDA_GATE_LOG_DECAY, o=None,
                    out_dtype=torch.float32, stream=None):
    """Outputs of T draft tokens per request from the checkpoint S (read only).
    q, k, g [N,T,H,dk]; v [N,T,H,dv]; beta [N,T,H]; S [N,H,dk,dv] float32.
    Returns o [N,T,H,dv]."""
    lib = _load()
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, T, H, dv), dtype=out_dtype, device=q.device)
    st = lib.kda_spec_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                             N, T, H, dk, dv, _dcode(q.dtype), _dcode(o.dtype), int(gate),
                             _stream(stream, q.device))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_spec_verify")
    return o


def kda_spec_commit(k, v, g, beta, S, accepted, *, gate=KDA_GATE_LOG_DECAY, stream=None):
    """Advance the checkpoint S [N,H,dk,dv] in place over the first accepted[n]
    (int32 [N] on the device) of the T logged tokens. Returns S."""
    lib = _load()
    N, T, H, dk = k.shape
    dv = v.shape[-1]
    if accepted.dtype != torch.int32:
        raise TypeError("accepted must be int32")
    st = lib.kda_spec_commit(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(accepted),
                             N, T, H, dk, dv, _dcode(k.dtype), int(gate), _stream(stream, k.device))
    if st != _STATUS_OK:
        raise KDAError(st, "kda_spec_commit")
    return S
