"""The prep stage on its own: the per-pair records that kda_chunk_prep writes
for bf16 inputs, decoded and compared part by part with the chunk form's
matrices (oracle.ref.chunk_terms, fp64), before any state pass runs.

A record holds, for chunks c1 and c2 of a pair (chunk form of the oracle
module; gamma1, gamma2 the chunks' total log-decays per channel):
  w1 = -W1, w2 = -W2 Diag(e^gamma1), q1 = Qt1, q2 = Qt2 Diag(e^gamma1),
  kb = [Kb1 Diag(e^gamma2) | Kb2], m1 = M1, [M21 | M2] with M21 = Qt2 Kb1^T,
  tb1 = Tb1, tb2 = Tb2 (Tb = Tm diag(beta)), c21 = -W2 Kb1^T,
  eg = e^(gamma1 + gamma2),
in the matrix-core fragment order the state pass reads: lane l (c16 = l % 16,
gq = l // 16) holds token c16 and channels 16m + 4gq + i of the dk-wide
operands; token 4gq + i and channel 16m + c16 of kb; entries [c16][4gq + i]
of the 16 x 16 tiles. The layout below is this test's own reading of that
order (the workspace is opaque to callers). Bar: the parts are fp16 (or a
bf16 or fp16 high/low pair), so each part must match to 4e-3 of its largest
entry, beyond an absolute floor of two fp16 subnormal steps.
"""
import numpy as np
import pytest
import torch

from gpucase import announce
from linear_attention_recurrence_11_amd import binding, inputs
from oracle import ref

pytestmark = pytest.mark.gpu
DEV = "cuda"
BAR = 4e-3
FLOOR = 2.0 ** -23  # two fp16 subnormal steps


def _layout(dk):
    tile = dk * 16 * 2
    L = dict(w1=0, w2=tile, q1=2 * tile, q2=3 * tile, kb=4 * tile, m1=6 * tile)
    L["m2h"] = L["m1"] + 1024
    L["m2l"] = L["m2h"] + 1024
    L["tb1"] = L["m2l"] + 1024
    L["tb2"] = L["tb1"] + 1024
    L["c21"] = L["tb2"] + 1024
    L["eg"] = L["c21"] + 512
    L["bytes"] = (L["eg"] + dk * 4 + 1023) // 1024 * 1024
    return L


def _f16(rec, off, n):
    return rec[off:off + 2 * n].view(np.float16).astype(np.float64)


def _bf16(rec, off, n):
    bits = rec[off:off + 2 * n].view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def _widen(a):
    """The oracle's input form (bf16 as raw 16-bit patterns) as exact float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _lanes():
    l = np.arange(64)
    return l % 16, l // 16


def _decode_rows(vals, dk):
    """[NM/2, 64, 8] fragment values -> [16 tokens, dk channels]."""
    c16, gq = _lanes()
    out = np.zeros((16, dk))
    for p in range(dk // 32):
        for j in range(8):
            out[c16, 16 * (2 * p + j // 4) + 4 * gq + j % 4] = vals[p, :, j]
    return out


def _decode_tile(vals):
    """[64, 4] fragment values -> 16 x 16 tile [c16][4gq + i]."""
    c16, gq = _lanes()
    out = np.zeros((16, 16))
    for i in range(4):
        out[c16, 4 * gq + i] = vals[:, i]
    return out


def _decode(rec, dk):
    L = _layout(dk)
    NM = dk // 16
    c16, gq = _lanes()
    d = {}
    for name in ("w1", "w2", "q1", "q2"):
        d[name] = _decode_rows(_f16(rec, L[name], 16 * dk).reshape(NM // 2, 64, 8), dk)
    kb = _f16(rec, L["kb"], 32 * dk).reshape(NM, 64, 8)
    d["kb1"], d["kb2"] = np.zeros((16, dk)), np.zeros((16, dk))
    for m in range(NM):
        for i in range(4):
            d["kb1"][4 * gq + i, 16 * m + c16] = kb[m, :, i]
            d["kb2"][4 * gq + i, 16 * m + c16] = kb[m, :, 4 + i]
    m1 = _f16(rec, L["m1"], 512).reshape(64, 8)
    d["m1"] = _decode_tile(m1[:, :4] + m1[:, 4:])
    m2 = _f16(rec, L["m2h"], 512).reshape(64, 8) + _f16(rec, L["m2l"], 512).reshape(64, 8)
    d["m21"], d["m2"] = _decode_tile(m2[:, :4]), _decode_tile(m2[:, 4:])
    for name in ("tb1", "tb2"):
        x = _bf16(rec, L[name], 512).reshape(64, 8)
        d[name] = _decode_tile(x[:, :4] + x[:, 4:])
    d["c21"] = _decode_tile(_f16(rec, L["c21"], 256).reshape(64, 4))
    eg = rec[L["eg"]:L["eg"] + 4 * dk].view(np.float32).astype(np.float64)
    d["eg"] = np.zeros(dk)
    for g4 in range(4):
        for m in range(NM):
            for i in range(4):
                d["eg"][16 * m + 4 * g4 + i] = eg[g4 * (dk // 4) + 4 * m + i]
    return d


def _chunk(x, t0, T):
    """Tokens [t0, t0 + 16) of one head, padded past T with the tokens that
    leave the state unchanged (q = k = g = beta = 0)."""
    q, k, g, beta = x
    out = []
    for a in (q, k, g):
        c = np.zeros((16, a.shape[1]))
        n = max(0, min(16, T - t0))
        c[:n] = a[t0:t0 + n]
        out.append(c)
    b = np.zeros(16)
    n = max(0, min(16, T - t0))
    b[:n] = beta[t0:t0 + n]
    out[2] = ref.clamp_decay(out[2])
    return ref.chunk_terms(out[0], out[1], out[2], b)


def _expected(c1, c2):
    e1, e2 = np.exp(c1["gam"]), np.exp(c2["gam"])
    return dict(w1=-c1["W"], w2=-c2["W"] * e1[None, :], q1=c1["Qt"], q2=c2["Qt"] * e1[None, :],
                kb1=c1["Kb"] * e2[None, :], kb2=c2["Kb"], m1=c1["M"], m2=c2["M"],
                m21=c2["Qt"] @ c1["Kb"].T, tb1=c1["Tb"], tb2=c2["Tb"], c21=-(c2["W"] @ c1["Kb"].T),
                eg=e1 * e2)


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("T", [64, 81], ids=["two_pairs", "ragged"])
def test_prep_records_match_the_chunk_form(dk, T):
    B, H, dv = 1, 2, 32
    ins = inputs.make_forward(B, T, H, dk, dv, "bf16", "normal", seed=95 + dk + T, device=DEV)
    announce("prep records", dk, T)
    ws = binding.kda_chunk_prep(ins["q"], ins["k"], ins["g"], ins["beta"], dv)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    L = _layout(dk)
    NPR = (T + 31) // 32
    host = {n: _widen(inputs.to_oracle(ins[n])) for n in ("q", "k", "g", "beta")}
    worst = 0.0
    for h in range(H):
        x = (host["q"][0, :, h], host["k"][0, :, h], host["g"][0, :, h], host["beta"][0, :, h])
        for s in range(NPR):
            rec = raw[(h * NPR + s) * L["bytes"]:(h * NPR + s + 1) * L["bytes"]]
            got = _decode(rec, dk)
            want = _expected(_chunk(x, 32 * s, T), _chunk(x, 32 * s + 16, T))
            for name, ref_val in want.items():
                scale = float(np.abs(ref_val).max())
                # fp16 spaces its subnormals 2^-24 apart: parts scaled by a
                # strong decay keep that absolute floor, not the relative bar
                excess = float(np.max(np.abs(got[name] - ref_val) - FLOOR))
                err = max(excess, 0.0) / (scale if scale > 0 else 1.0)
                worst = max(worst, err)
                assert err <= BAR, (h, s, name, err)
    announce("  worst part error %.3g" % worst)
