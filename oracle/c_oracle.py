"""ctypes wrapper around the C fp64 oracle (kda_oracle.c).

Test infrastructure: see the package docstring. Inputs are NumPy arrays of
float32 or of bfloat16 bit patterns (uint16); they are widened to double
exactly inside the C code. Outputs are float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
F32, BF16 = 0, 1
GATE_LOG_DECAY, GATE_SIGMOID = 0, 1


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        vp, l, i = ctypes.c_void_p, ctypes.c_long, ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, vp, vp, vp, l, l, l, l, l, i]
        lib.kda_oracle_fwd.restype = i
        lib.kda_oracle_fwd_cols.argtypes = [vp, vp, vp, vp, vp, i, i, l, l, l, l, l, l, l,
                                            vp, l, vp, vp, vp]
        lib.kda_oracle_fwd_cols.restype = i
        _lib = lib
    return _lib


def _dtype_code(arrs):
    dts = {a.dtype for a in arrs}
    if dts == {np.dtype(np.float32)}:
        return F32
    if dts == {np.dtype(np.uint16)}:
        return BF16
    raise TypeError("oracle inputs must all be float32 or all be bfloat16 bits (uint16), got %s" % dts)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def fwd(q, k, v, g, beta, S0=None, nthreads=None, want_o=True, want_state=True, gate=GATE_LOG_DECAY):
    """Sequential fp64 recurrence. Shapes: q,k,g [B,T,H,dk]; v [B,T,H,dv];
    beta [B,T,H]; S0 [B,H,dk,dv] (any float dtype, widened to double) or None.
    gate=GATE_SIGMOID reads g as gate logits x with log-decay -5 sigmoid(x).
    Returns (o [B,T,H,dv] float64 or None, S_T [B,H,dk,dv] float64 or None)."""
    q, k, v, g, beta = (np.ascontiguousarray(x) for x in (q, k, v, g, beta))
    code = _dtype_code([q, k, v, g, beta])
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, T, H, dv)
    assert beta.shape == (B, T, H)
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, dtype=np.float64)
        assert s0.shape == (B, H, dk, dv)
    o = np.empty((B, T, H, dv), np.float64) if want_o else None
    st = np.empty((B, H, dk, dv), np.float64) if want_state else None
    rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), code, int(gate),
                                _ptr(s0), _ptr(o), _ptr(st), B, T, H, dk, dv,
                                int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments (code %d)" % rc)
    return o, st


def fwd_cols(q, k, v, g, beta, b, h, cols, S0c=None, gate=GATE_LOG_DECAY):
    """The recurrence for one (b, h) restricted to value columns `cols`.
    Returns (o_cols [T, ncols], S_T cols [dk, ncols]) in float64."""
    q, k, v, g, beta = (np.ascontiguousarray(x) for x in (q, k, v, g, beta))
    code = _dtype_code([q, k, v, g, beta])
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    n = cols.size
    s0 = None if S0c is None else np.ascontiguousarray(S0c, dtype=np.float64)
    if s0 is not None:
        assert s0.shape == (dk, n)
    oc = np.empty((T, n), np.float64)
    stc = np.empty((dk, n), np.float64)
    rc = _load().kda_oracle_fwd_cols(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), code,
                                     int(gate), B, T, H, dk, dv, int(b), int(h), _ptr(cols), n,
                                     _ptr(s0), _ptr(oc), _ptr(stc))
    if rc != 0:
        raise ValueError("kda_oracle_fwd_cols rejected its arguments (code %d)" % rc)
    return oc, stc
