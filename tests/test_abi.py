"""The C-ABI library loads on the CPU and exports every symbol include/kda.h
declares; host-side argument checks behave as documented (no GPU used: only
calls that are rejected before any HIP call, and the pure host functions)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_11_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
OK, NULL, SHAPE, UNSUP, ALIAS, WS, HIP, ALIGN, TOO_LARGE = range(9)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from linear_attention_recurrence_11_amd import build
        build.build()
    return binding._load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "libkda.so does not export %s" % n


def test_version_and_status_strings(lib):
    assert binding.kda_abi_version() == binding.ABI_VERSION == 4
    for s in range(9):
        assert binding.kda_status_str(s) and binding.kda_status_str(s) != "unknown status"
    assert binding.kda_status_str(99) == "unknown status"


def test_workspace_size(lib):
    # fp32 inputs: one record per (b, h, 16-token chunk), whole KiB: 27648 B
    # (dk 128), 15360 B (dk 64); bf16 inputs: one per (b, h, pair of chunks):
    # 30720 B (dk 128), 18432 B (dk 64), then a 4-byte flag per (b, h, 16
    # columns of dk + dv: the transition's F and E run as one pass), rounded up
    # to whole KiB
    assert binding.kda_chunk_fwd_workspace_size(1, 65536, 32, 128, 128, BF16) == \
        32 * 2048 * 30720 + 2048
    assert binding.kda_chunk_fwd_workspace_size(4, 4096, 16, 128, 128, BF16) == \
        64 * 128 * 30720 + 4096
    assert binding.kda_chunk_fwd_workspace_size(1, 33, 2, 64, 64, BF16) == 2 * 2 * 18432 + 1024
    assert binding.kda_chunk_fwd_workspace_size(1, 256, 2, 64, 64, F32) == 2 * 16 * 15360
    assert binding.kda_chunk_fwd_workspace_size(1, 17, 1, 128, 128, F32) == 2 * 27648
    assert binding.kda_chunk_fwd_workspace_size(1, 0, 1, 128, 128, F32) == 0
    assert binding.kda_chunk_fwd_workspace_size(1, 16, 1, 96, 128, F32) == 0
    assert binding.kda_chunk_fwd_workspace_size(1, 16, 1, 128, 24, F32) == 0


BASE = 1 << 40   # fake, never dereferenced, 16-byte aligned addresses


def fake_chunk(B=1, T=32, H=2, dk=64, dv=64, ind=F32, outd=F32, s0=True, st=True, ws=True):
    es = 4 if ind == F32 else 2
    n = B * T * H
    off = [BASE]

    def alloc(nbytes):
        p = off[0]
        off[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p
    p = dict(q=alloc(n * dk * es), k=alloc(n * dk * es), v=alloc(n * dv * es),
             g=alloc(n * dk * es), beta=alloc(n * es),
             S0=alloc(B * H * dk * dv * 4) if s0 else None,
             o=alloc(n * dv * (4 if outd == F32 else 2)),
             S_T=alloc(B * H * dk * dv * 4) if st else None)
    need = binding.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, ind)
    p["ws"] = alloc(need) if ws else None
    p["ws_bytes"] = need
    return p, (B, T, H, dk, dv, ind, outd)


def check(lib, p, sizes, **over):
    p = dict(p)
    p.update(over)
    B, T, H, dk, dv, ind, outd = sizes
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return lib.kda_chunk_fwd_check(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]), vp(p["beta"]),
                                   vp(p["S0"]), vp(p["o"]), vp(p["S_T"]), B, T, H, dk, dv, ind,
                                   outd, vp(p["ws"]), p["ws_bytes"])


def test_chunk_check_accepts_valid(lib):
    for kw in (dict(), dict(ind=BF16), dict(ind=BF16, outd=BF16, dk=128, dv=128),
               dict(dv=16), dict(dv=512), dict(T=1), dict(T=17), dict(s0=False, st=False)):
        p, sz = fake_chunk(**kw)
        assert check(lib, p, sz) == OK, kw


def test_chunk_check_rejects(lib):
    p, sz = fake_chunk()
    assert check(lib, p, sz, q=None) == NULL
    assert check(lib, p, sz, o=None) == NULL
    assert check(lib, p, sz, ws=None) == WS
    assert check(lib, p, sz, ws_bytes=p["ws_bytes"] - 1) == WS
    assert check(lib, p, sz, q=p["q"] + 8) == ALIGN         # fp32 q: 4-element vectors
    assert check(lib, p, sz, ws=p["ws"] + 8) == ALIGN
    assert check(lib, p, sz, beta=p["beta"] + 2) == ALIGN
    assert check(lib, p, sz, beta=p["beta"] + 4) == OK      # element-aligned is enough
    assert check(lib, p, sz, o=p["o"] + 4) == ALIGN         # forward o: 16 bytes
    assert check(lib, p, sz, o=p["o"] + 16) == OK
    assert check(lib, p, sz, o=p["q"]) == ALIAS            # o over q
    assert check(lib, p, sz, o=p["S0"]) == ALIAS           # o over S0
    assert check(lib, p, sz, S_T=p["S0"] + 64) == ALIAS    # partial state overlap
    assert check(lib, p, sz, S_T=p["S0"]) == OK            # exact alias: in place
    assert check(lib, p, sz, ws=p["v"]) == ALIAS           # workspace over v
    B, T, H, dk, dv, ind, outd = sz
    assert check(lib, p, (B, -1, H, dk, dv, ind, outd)) == SHAPE
    assert check(lib, p, (B, T, H, 96, dv, ind, outd)) == UNSUP
    assert check(lib, p, (B, T, H, dk, 24, ind, outd)) == UNSUP
    assert check(lib, p, (B, T, H, dk, 528, ind, outd)) == UNSUP
    assert check(lib, p, (B, T, H, dk, dv, 7, outd)) == UNSUP
    assert check(lib, p, (B, T, H, dk, dv, ind, 5)) == UNSUP


def test_chunk_empty_needs_nothing(lib):
    p, sz = fake_chunk()
    B, T, H, dk, dv, ind, outd = sz
    nulls = dict(q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, ws_bytes=0)
    assert check(lib, p, (B, 0, H, dk, dv, ind, outd), **nulls) == OK
    assert check(lib, p, (0, T, H, dk, dv, ind, outd), **nulls) == OK


def test_chunk_empty_sequence_with_huge_batch_and_heads(lib):
    # T = 0 puts no bound on B and H through the token count; B * H = 2^80
    # must be rejected without forming the product in 64-bit integers
    p, sz = fake_chunk()
    B, T, H, dk, dv, ind, outd = sz
    nulls = dict(q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, ws_bytes=0,
                 S0=None, S_T=None)
    assert check(lib, p, (1 << 40, 0, 1 << 40, dk, dv, ind, outd), **nulls) == UNSUP
    assert check(lib, p, (1 << 14, 0, 1 << 14, dk, dv, ind, outd), **nulls) == UNSUP  # 2^28
    assert check(lib, p, (1 << 13, 0, 1 << 14, dk, dv, ind, outd), **nulls) == OK


def test_chunk_fwd_rejects_before_any_launch(lib):
    """kda_chunk_fwd returns the check's error without touching the GPU."""
    p, sz = fake_chunk()
    B, T, H, dk, dv, ind, outd = sz
    vp = ctypes.c_void_p
    st = lib.kda_chunk_fwd(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]), vp(p["beta"]),
                           vp(p["S0"]), vp(p["q"]), vp(p["S_T"]), B, T, H, dk, dv, ind, outd,
                           vp(p["ws"]), p["ws_bytes"], None)
    assert st == ALIAS
    st = lib.kda_chunk_fwd(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]), vp(p["beta"]),
                           vp(p["S0"]), vp(p["o"]), vp(p["S_T"]), B, T, H, 80, dv, ind, outd,
                           vp(p["ws"]), p["ws_bytes"], None)
    assert st == UNSUP
    # empty work returns OK without a launch
    st = lib.kda_chunk_fwd(None, None, None, None, None, None, None, None, 0, 5, 3, 64, 64, 0, 0,
                           None, 0, None)
    assert st == OK


def test_decode_check(lib):
    vp = ctypes.c_void_p
    N, H, dk, dv = 4, 2, 128, 128
    a = [BASE + i * (1 << 24) for i in range(7)]   # q k v g beta S o
    call = lambda ptrs, N=N, H=H, dk=dk, dv=dv, ind=BF16, outd=F32: lib.kda_decode_step_check(
        *[vp(x) if x is not None else None for x in ptrs], N, H, dk, dv, ind, outd)
    assert call(a) == OK
    assert call(a, dk=64, dv=64) == OK
    assert call(a, dv=96) == UNSUP
    assert call(a[:6] + [a[5]]) == ALIAS        # o over S
    assert call(a[:5] + [a[0]] + [a[6]]) == ALIAS   # S over q
    assert call([None] + a[1:]) == NULL
    assert call(a[:6] + [a[6] + 2]) == ALIGN                # fp32 o
    assert call(a[:6] + [a[6] + 4]) == OK
    assert call(a[:5] + [a[5] + 8] + [a[6]]) == ALIGN       # state: 16 bytes
    assert call([a[0] + 2] + a[1:]) == OK                    # bf16 q: element-aligned
    assert call(a, N=-1) == SHAPE
    assert call([None] * 7, N=0) == OK
    st = lib.kda_decode_step(*[vp(x) for x in a[:6]], vp(a[5]), N, H, dk, dv, BF16, F32, None)
    assert st == ALIAS


def test_stage_entry_points_check_their_own_tensors(lib):
    p, sz = fake_chunk()
    B, T, H, dk, dv, ind, outd = sz
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    prep = lambda **o: lib.kda_chunk_prep(
        vp(o.get("q", p["q"])), vp(p["k"]), vp(p["g"]), vp(p["beta"]), B, o.get("T", T), H, dk, dv,
        ind, vp(o.get("ws", p["ws"])), o.get("ws_bytes", p["ws_bytes"]), None)
    passf = lambda **o: lib.kda_chunk_state_pass(
        vp(o.get("v", p["v"])), vp(o.get("ws", p["ws"])), p["ws_bytes"], vp(p["S0"]),
        vp(o.get("o", p["o"])), vp(o.get("S_T", p["S_T"])), B, T, H, dk, dv, ind, outd, None)
    assert prep(q=None) == NULL
    assert prep(ws=None) == WS
    assert prep(ws_bytes=p["ws_bytes"] - 16) == WS
    assert prep(ws=p["q"]) == ALIAS
    assert prep(q=p["q"] + 4) == ALIGN
    assert prep(T=0, ws=None, ws_bytes=0) == OK       # nothing to do, no launch
    assert passf(v=None) == NULL
    assert passf(o=p["v"]) == ALIAS
    assert passf(ws=p["o"]) == ALIAS
    assert passf(S_T=p["S0"] + 128) == ALIAS
    assert passf(v=p["v"] + 2) == ALIGN
    assert passf(v=p["v"] + 8) == ALIGN      # v: 16 bytes


def check_ex(lib, p, sizes, gate=0, snaps=None, every=0, **over):
    p = dict(p)
    p.update(over)
    B, T, H, dk, dv, ind, outd = sizes
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return lib.kda_chunk_fwd_ex_check(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]), vp(p["beta"]),
                                      vp(p["S0"]), vp(p["o"]), vp(p["S_T"]), B, T, H, dk, dv, ind,
                                      outd, gate, vp(snaps), every, vp(p["ws"]), p["ws_bytes"])


def test_chunk_ex_check_gate_and_snapshots(lib):
    p, sz = fake_chunk(T=1040)           # 1040 = 2 * 512 + 16: two snapshots at every = 512
    snaps = BASE + (1 << 36)             # far from every other fake tensor
    assert check_ex(lib, p, sz) == OK
    assert check_ex(lib, p, sz, gate=1) == OK
    assert check_ex(lib, p, sz, gate=2) == UNSUP
    assert check_ex(lib, p, sz, snaps=snaps, every=512) == OK
    assert check_ex(lib, p, sz, snaps=snaps, every=32) == OK
    assert check_ex(lib, p, sz, snaps=snaps, every=16) == UNSUP   # whole 32-token steps
    assert check_ex(lib, p, sz, snaps=None, every=512) == NULL
    assert check_ex(lib, p, sz, snaps=None, every=2048) == OK      # none falls inside T
    assert check_ex(lib, p, sz, snaps=snaps, every=-16) == SHAPE
    assert check_ex(lib, p, sz, snaps=snaps, every=500) == UNSUP
    assert check_ex(lib, p, sz, snaps=snaps + 2, every=512) == ALIGN
    assert check_ex(lib, p, sz, snaps=p["o"], every=512) == ALIAS
    assert check_ex(lib, p, sz, snaps=p["S0"], every=512) == ALIAS
    assert check_ex(lib, p, sz, snaps=p["ws"], every=512) == ALIAS
    # the plain checks still apply
    assert check_ex(lib, p, sz, o=p["q"]) == ALIAS
    vp = ctypes.c_void_p
    B, T, H, dk, dv, ind, outd = sz
    st = lib.kda_chunk_fwd_ex(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]), vp(p["beta"]),
                              vp(p["S0"]), vp(p["o"]), vp(p["S_T"]), B, T, H, dk, dv, ind, outd,
                              3, None, 0, vp(p["ws"]), p["ws_bytes"], None)
    assert st == UNSUP


def test_decode_ex_rejects_unknown_gate(lib):
    vp = ctypes.c_void_p
    a = [BASE + i * (1 << 24) for i in range(7)]
    st = lib.kda_decode_step_ex(*[vp(x) for x in a], 4, 2, 128, 128, BF16, F32, 5, None)
    assert st == UNSUP
    st = lib.kda_decode_step_ex(*[vp(x) for x in a[:6]], vp(a[5]), 4, 2, 128, 128, BF16, F32, 1,
                                None)
    assert st == ALIAS


def test_spec_checks(lib):
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    N, T, H, dk, dv = 3, 4, 2, 128, 64
    a = [BASE + i * (1 << 24) for i in range(8)]   # q k v g beta S o accepted
    ver = lambda ptrs, T=T, dv=dv, gate=0: lib.kda_spec_verify_check(
        *[vp(x) for x in ptrs[:7]], N, T, H, dk, dv, BF16, F32, gate)
    com = lambda ptrs, T=T, gate=0: lib.kda_spec_commit_check(
        *[vp(x) for x in ptrs[1:6] + [ptrs[7]]], N, T, H, dk, dv, BF16, gate)
    assert ver(a) == OK and com(a) == OK
    assert ver(a, gate=1) == OK and com(a, gate=1) == OK
    assert ver(a, gate=2) == UNSUP and com(a, gate=9) == UNSUP
    assert ver(a, dv=96) == UNSUP
    assert ver([None] + a[1:]) == NULL                        # verify reads q
    assert com([None] + a[1:]) == OK                          # commit does not
    assert com(a[:7] + [None]) == NULL                        # commit needs accepted
    assert ver(a[:6] + [a[5]] + a[7:]) == ALIAS               # o over the checkpoint
    assert ver(a[:6] + [a[1]] + a[7:]) == ALIAS               # o over k
    assert com(a[:5] + [a[2]] + a[6:]) == ALIAS               # S over v
    assert com(a[:7] + [a[5]]) == ALIAS                       # accepted over S
    assert ver(a[:5] + [a[5] + 8] + a[6:]) == ALIGN           # state: 16 bytes
    assert com(a[:7] + [a[7] + 2]) == ALIGN                   # accepted: 4 bytes
    assert ver([None] * 8, T=0) == OK and com([None] * 8, T=0) == OK
    st = lib.kda_spec_verify(*[vp(x) for x in a[:6]], vp(a[5]), N, T, H, dk, dv, BF16, F32, 0, None)
    assert st == ALIAS
    st = lib.kda_spec_commit(*[vp(x) for x in a[1:5]], vp(a[5]), vp(a[5]), N, T, H, dk, dv, BF16, 0,
                             None)
    assert st == ALIAS


def test_spec_commit_verify_checks(lib):
    # the fused round boundary: each step's rules, and across the two token
    # sets S (written) off the drafts and o off the logged tokens
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    N, H, dk, dv = 3, 2, 128, 64
    names = ["k1", "v1", "g1", "beta1", "acc", "q2", "k2", "v2", "g2", "beta2", "S", "o"]
    base = {n: BASE + i * (1 << 24) for i, n in enumerate(names)}

    def cv(T1=4, T2=5, gate=0, **over):
        p = dict(base, **over)
        return lib.kda_spec_commit_verify_check(
            *[vp(p[n]) for n in names[:5]], T1, *[vp(p[n]) for n in names[5:10]], T2,
            vp(p["S"]), vp(p["o"]), N, H, dk, dv, BF16, F32, gate)

    assert cv() == OK and cv(gate=1) == OK
    assert cv(gate=3) == UNSUP
    assert cv(acc=None) == NULL                      # the commit needs accepted
    assert cv(q2=None) == NULL                       # the verify reads q
    assert cv(T1=0, k1=None, v1=None, g1=None, beta1=None, acc=None) == OK   # a plain verify
    assert cv(T2=0, q2=None, k2=None, v2=None, g2=None, beta2=None, o=None) == OK  # a plain commit
    assert cv(T1=0, T2=0, **{n: None for n in names}) == OK
    assert cv(S=base["v1"]) == ALIAS                 # S over a logged input
    assert cv(S=base["k2"]) == ALIAS                 # S over a draft
    assert cv(o=base["S"]) == ALIAS                  # o over the state
    assert cv(o=base["g1"]) == ALIAS                 # o over a logged input
    assert cv(o=base["acc"]) == ALIAS                # o over the accepted counts
    assert cv(o=base["v2"]) == ALIAS                 # o over a draft
    assert cv(S=base["S"] + 8) == ALIGN              # the state: 16 bytes
    assert cv(acc=base["acc"] + 2) == ALIGN          # accepted: 4 bytes
    assert cv(k2=base["k2"] + 2) == OK               # inputs: element alignment only
    st = lib.kda_spec_commit_verify(*[vp(base[n]) for n in names[:5]], 4,
                                    *[vp(base[n]) for n in names[5:10]], 5, vp(base["S"]),
                                    vp(base["S"]), N, H, dk, dv, BF16, F32, 0, None)
    assert st == ALIAS                               # checked before any launch


def test_transition_and_scan_checks(lib):
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    p, sz = fake_chunk(B=2, T=40, H=3, dk=128, dv=64, ind=BF16)
    B, T, H, dk, dv, ind, _ = sz
    F = BASE + (1 << 36)
    E = F + (1 << 30)
    tr = lambda **o: lib.kda_chunk_transition_check(
        vp(o.get("v", p["v"])), vp(o.get("ws", p["ws"])), o.get("ws_bytes", p["ws_bytes"]),
        vp(o.get("F", F)), vp(o.get("E", E)), B, o.get("T", T), H, o.get("dk", dk), dv, ind)
    assert tr() == OK
    assert tr(E=None, v=None) == OK                 # F alone reads no v
    assert tr(v=None) == NULL                       # E needs v
    assert tr(F=None, E=None, ws=None, ws_bytes=0) == OK
    assert tr(ws_bytes=p["ws_bytes"] - 1) == WS
    assert tr(E=F + 64) == ALIAS
    assert tr(F=p["ws"]) == ALIAS
    assert tr(E=p["v"]) == ALIAS
    assert tr(F=F + 2) == ALIGN
    assert tr(v=p["v"] + 8) == ALIGN
    assert tr(dk=96) == UNSUP
    assert tr(T=-1) == SHAPE
    assert tr(T=0, ws=None, ws_bytes=0, v=None) == OK
    # the workspace also holds one flag per 16 columns of dk + dv
    assert binding.kda_chunk_fwd_workspace_size(1, 32, 64, 128, 16, BF16) == \
        64 * 30720 + (64 * 9 * 4 + 1023) // 1024 * 1024
    sc = lambda P=3, N=4, dk=128, dv=64, **o: lib.kda_state_affine_scan_check(
        vp(o.get("F", F)), vp(o.get("E", E)), vp(o.get("S0", BASE)), vp(o.get("S", BASE + (1 << 38))),
        P, N, dk, dv)
    assert sc() == OK
    assert sc(S0=None) == OK
    assert sc(F=None) == NULL and sc(S=None) == NULL
    assert sc(P=0, F=None, E=None) == OK
    assert sc(S=F) == ALIAS and sc(S=BASE) == ALIAS
    assert sc(F=F + 4) == ALIGN                     # F is read as 4-float vectors
    assert sc(dk=96) == UNSUP and sc(dv=40) == UNSUP
    assert sc(P=-1) == SHAPE
    st = lib.kda_state_affine_scan(vp(F), vp(E), None, vp(F), 3, 4, 128, 64, None)
    assert st == ALIAS


def test_noalloc_check(lib):
    """The no-allocation forward applies the forward's checks and rejects
    work beyond its built-in scratch before anything runs."""
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    limit = binding.NOALLOC_SCRATCH_BYTES

    def chk(p, sz, **over):
        p = dict(p)
        p.update(over)
        B, T, H, dk, dv, ind, outd = sz
        return lib.kda_chunk_fwd_noalloc_check(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]),
                                               vp(p["beta"]), vp(p["S0"]), vp(p["o"]),
                                               vp(p["S_T"]), B, T, H, dk, dv, ind, outd)
    p, sz = fake_chunk(B=1, T=2048, H=32, dk=128, dv=128, ind=BF16, ws=False)
    assert binding.kda_chunk_fwd_workspace_size(1, 2048, 32, 128, 128, BF16) <= limit
    assert chk(p, sz) == OK
    assert chk(p, sz, o=p["q"]) == ALIAS
    assert chk(p, sz, q=None) == NULL
    p2, sz2 = fake_chunk(B=1, T=4096, H=32, dk=128, dv=128, ind=BF16, ws=False)
    assert binding.kda_chunk_fwd_workspace_size(1, 4096, 32, 128, 128, BF16) > limit
    assert chk(p2, sz2) == TOO_LARGE
    assert "scratch" in binding.kda_status_str(TOO_LARGE)
    B, T, H, dk, dv, ind, outd = sz2
    st = lib.kda_chunk_fwd_noalloc(vp(p2["q"]), vp(p2["k"]), vp(p2["v"]), vp(p2["g"]),
                                   vp(p2["beta"]), vp(p2["S0"]), vp(p2["o"]), vp(p2["S_T"]),
                                   B, T, H, dk, dv, ind, outd, None)
    assert st == TOO_LARGE                          # rejected on the host, nothing launched
    empty = lib.kda_chunk_fwd_noalloc(None, None, None, None, None, None, None, None,
                                      0, 5, 3, 64, 64, BF16, F32, None)
    assert empty == OK


def test_injected_launch_failures(lib):
    """A call that passes its checks takes an injected failure and returns
    KDA_ERR_HIP without any HIP call (every call here uses fake pointers and
    must not launch); a call that fails its checks reports that first and
    leaves the count alone."""
    vp = ctypes.c_void_p
    a = [BASE + i * (1 << 24) for i in range(7)]   # q k v g beta S o
    dec = lambda o=a[6]: lib.kda_decode_step(*[vp(x) for x in a[:6]], vp(o), 4, 2, 128, 128, BF16,
                                             F32, None)
    try:
        binding.kda_debug_inject_launch_failures(2)
        assert dec() == HIP
        assert dec(o=a[5]) == ALIAS                 # checks first; count untouched
        assert dec() == HIP                         # the second injected failure
        binding.kda_debug_inject_launch_failures(1)
        p, sz = fake_chunk()
        B, T, H, dk, dv, ind, outd = sz
        st = lib.kda_chunk_fwd(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]), vp(p["beta"]),
                               vp(p["S0"]), vp(p["o"]), vp(p["S_T"]), B, T, H, dk, dv, ind, outd,
                               vp(p["ws"]), p["ws_bytes"], None)
        assert st == HIP
        binding.kda_debug_inject_launch_failures(1)
        F = BASE + (1 << 36)
        st = lib.kda_state_affine_scan(vp(F), vp(F + (1 << 30)), None, vp(F + (1 << 31)), 2, 3,
                                       128, 64, None)
        assert st == HIP
        binding.kda_debug_inject_launch_failures(1)
        st = lib.kda_chunk_fwd_noalloc(vp(p["q"]), vp(p["k"]), vp(p["v"]), vp(p["g"]),
                                       vp(p["beta"]), vp(p["S0"]), vp(p["o"]), vp(p["S_T"]),
                                       B, T, H, dk, dv, ind, outd, None)
        assert st == HIP                            # taken before the scratch lookup
    finally:
        binding.kda_debug_inject_launch_failures(0)
