"""Host checks of the tiled int4 code layout's definition (no GPU).

The definition (C header, tiled code layout) must be a byte permutation of
the plain codes, keep every 16-byte run of a row intact, and put the 64
lane-runs of one (tile, group) in 1 KiB of contiguous memory. A hand-worked
position pins the index order.
"""
import numpy as np
import pytest

from helpers import tiled_codes


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_tiled_is_a_byte_permutation(kind):
    rng = np.random.default_rng(kind)
    E, N, K2 = 2, 256, 128            # N = 2I for w13 (I = 128), K = 256 (2 groups)
    # every byte position gets a distinct 32-bit tag -> track where it goes
    tags = np.arange(E * N * K2, dtype=np.int64).reshape(E, N, K2)
    lo = (tags & 0xFF).astype(np.uint8)
    hi = ((tags >> 8) & 0xFF).astype(np.uint8)
    hh = ((tags >> 16) & 0xFF).astype(np.uint8)
    t_lo, t_hi, t_hh = (tiled_codes(x, kind, N // 2) for x in (lo, hi, hh))
    back = t_lo.astype(np.int64) | (t_hi.astype(np.int64) << 8) | (t_hh.astype(np.int64) << 16)
    assert np.array_equal(np.sort(back.ravel()), tags.ravel())
    # within an expert, bytes stay inside that expert
    for e in range(E):
        assert (back[e] // (N * K2) == e).all()
    # 16-byte runs stay intact (consecutive bytes of one row)
    runs = back.reshape(-1, 16)
    assert (np.diff(runs, axis=1) == 1).all()
    _ = rng


def test_tiled_hand_worked_position():
    # W13_SWIGLU, I = 128: tile t = 3 holds gate rows 24..31 (lanes n = 0..7)
    # and up rows 128+24..128+31 (n = 8..15). Lane l = 16*kq + n of group g
    # is 16 bytes at plain byte offset 64g + 16kq of that row; its place is
    # block b = 0, i = 3, at ((b*G + g)*8 + i)*1024 + l*16 within the expert.
    E, N, K2 = 1, 256, 128
    G = 2
    plain = np.zeros((E, N, K2), np.uint8)
    row, g, kq, n = 128 + 24 + 5, 1, 2, 13            # up row of n = 13 in tile 3
    plain[0, row, 64 * g + 16 * kq: 64 * g + 16 * kq + 16] = np.arange(1, 17)
    t = tiled_codes(plain, 0, 128).reshape(-1)
    pos = ((0 * G + g) * 8 + 3) * 1024 + (16 * kq + n) * 16
    assert np.array_equal(t[pos:pos + 16], np.arange(1, 17))
    assert int(t.astype(np.int64).sum()) == int(np.arange(1, 17).sum())
