"""Host-side model of the two ways the bf16 state pass writes its V^T tiles.

With one or two slices per workgroup a loader lane (a = l % 16, cq = l // 16)
loads, per slice z, four columns 16z + 4cq .. + 3 of tokens 2a and 2a + 1 and
writes one dword (even token low, odd token high) per column into tile
2z + (a >> 3) at row 4cq + c, dword a & 7.

With two or four slices the V loads cover whole rows instead (VRows in the
kernel source). Four slices: in load i (0..3), lane l takes the 16 bytes of
columns 8j .. 8j + 7 (j = l & 7) of token 8i + (l >> 3). Two slices: in load
i (0..1), piece j = l & 3 of token 16i + (b3 + 2 b2 + 4 b4 + 8 b5), b the bits
of l. Either way lanes l and l ^ 8 (a DPP rotation by 8 within a 16-lane row)
hold tokens t and t ^ 1 and swap half their pieces, and each writes four
columns of the pair.

Both must produce the same tiles, including for tokens past the end of the
sequence (zeros). The model restates the kernel's index arithmetic."""
import numpy as np
import pytest


def per_slice_tiles(v, ok, spw=4):
    tiles = {}
    for l in range(64):
        a, cq = l & 15, l >> 4
        for z in range(spw):
            for c in range(4):
                col = 16 * z + 4 * cq + c
                lo = v[2 * a, col] if ok[2 * a] else 0
                hi = v[2 * a + 1, col] if ok[2 * a + 1] else 0
                key = (2 * z + (a >> 3), 4 * cq + c, a & 7)
                assert key not in tiles
                tiles[key] = int(lo) | (int(hi) << 16)
    return tiles


def _lane(l, i, spw):
    if spw == 4:
        return l & 7, 8 * i + (l >> 3)
    return l & 3, 16 * i + (((l >> 3) & 1) | (((l >> 2) & 1) << 1) | ((l >> 4) << 2))


def whole_row_tiles(v, ok, rotate=8, spw=4):
    tiles = {}
    for i in range(spw):
        mine = np.zeros((64, 4), dtype=np.uint64)
        for l in range(64):
            j, t = _lane(l, i, spw)
            if ok[t]:
                for d in range(4):
                    mine[l, d] = int(v[t, 8 * j + 2 * d]) | (int(v[t, 8 * j + 2 * d + 1]) << 16)
        odd = [(l >> 3) & 1 for l in range(64)]
        send = np.array([[mine[l, d] if odd[l] else mine[l, 2 + d] for d in range(2)] for l in range(64)])
        recv = np.array([send[(l // 16) * 16 + ((l % 16) + rotate) % 16] for l in range(64)])
        for l in range(64):
            j, t = _lane(l, i, spw)
            c0 = 8 * (j & 1) + (4 if odd[l] else 0)
            for k in range(4):
                d = k >> 1
                ew = int(recv[l, d] if odd[l] else mine[l, d])
                ow = int(mine[l, 2 + d] if odd[l] else recv[l, d])
                e = (ew >> 16) if (k & 1) else (ew & 0xFFFF)
                o = (ow & 0xFFFF0000) if (k & 1) else ((ow << 16) & 0xFFFFFFFF)
                key = (2 * (j >> 1) + (t >> 4), c0 + k, (t & 15) >> 1)
                assert key not in tiles
                tiles[key] = e | o
    return tiles


@pytest.mark.parametrize("spw", [2, 4])
@pytest.mark.parametrize("valid", [32, 31, 17, 16, 1])
def test_whole_row_loads_write_the_same_tiles(valid, spw):
    rng = np.random.default_rng(valid + spw)
    v = rng.integers(1, 1 << 16, size=(32, 16 * spw), dtype=np.uint32)  # bf16 bits, a pair's rows
    ok = np.arange(32) < valid
    a, b = per_slice_tiles(v, ok, spw), whole_row_tiles(v, ok, spw=spw)
    assert len(a) == spw * 2 * 16 * 8 and a == b


@pytest.mark.parametrize("spw", [2, 4])
def test_a_wrong_partner_lane_is_caught(spw):
    # the model has teeth: swapping with the lane 4 away pairs the wrong tokens
    rng = np.random.default_rng(0)
    v = rng.integers(1, 1 << 16, size=(32, 16 * spw), dtype=np.uint32)
    ok = np.ones(32, dtype=bool)
    assert per_slice_tiles(v, ok, spw) != whole_row_tiles(v, ok, rotate=4, spw=spw)
