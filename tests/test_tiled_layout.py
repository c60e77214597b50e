"""Host checks of the tiled int4 code layout's definition (no GPU).

The definition (C header, tiled code layout) must be a permutation of the
plain codes (4-bit units), keep the 8 codes of every plain 4-byte word in one
tiled word and the words of every 16-byte run of a row in one 16-byte run,
and put the 64 lane-runs of one (tile, group) in 1 KiB of contiguous memory.
Hand-worked positions pin the index order and the word shuffle.
"""
import numpy as np
import pytest

from helpers import shuffle_words, tiled_codes


def _nibbles(b):
    b = np.asarray(b, np.uint8)
    return np.stack([b & 0xF, b >> 4], axis=-1).reshape(*b.shape[:-1], -1)


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_tiled_is_a_code_permutation(kind):
    E, N, K2 = 2, 256, 128            # N = 2I for w13 (I = 128), K = 256 (2 groups)
    n_codes = E * N * K2 * 2
    # tag every code position with a distinct integer, carried by 5 nibble planes
    tags = np.arange(n_codes, dtype=np.int64).reshape(E, N, 2 * K2)
    back = np.zeros((E, N, 2 * K2), np.int64)
    for p in range(5):                                 # 20 bits cover 2^17 codes
        nib = ((tags >> (4 * p)) & 0xF).astype(np.uint8)
        packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
        back |= _nibbles(tiled_codes(packed, kind, N // 2)).astype(np.int64) << (4 * p)
    assert np.array_equal(np.sort(back.ravel()), tags.ravel())
    for e in range(E):                                  # codes stay inside their expert
        assert (back[e] // (N * 2 * K2) == e).all()
    # every tiled word holds the 8 codes of one plain word, every 16-byte run
    # the 32 codes of one plain 16-byte run
    words = back.reshape(-1, 8)
    assert (np.ptp(words // 8, axis=1) == 0).all()
    runs = back.reshape(-1, 32)
    assert (np.ptp(runs // 32, axis=1) == 0).all()


def test_word_shuffle_hand_worked():
    # plain word with codes c_j = j + 1 (c0 in the low nibble of byte 0):
    # bytes 0x21, 0x43, 0x65, 0x87. Even codes 1,3,5,7 go to nibbles 0..3,
    # odd codes 2,4,6,8 to nibbles 4..7: word 0x86427531.
    b = np.array([0x21, 0x43, 0x65, 0x87], np.uint8)
    assert shuffle_words(b).view("<u4")[0] == 0x86427531
    # nibble pair (j, j + 4) of the shuffled word = columns (2j, 2j + 1)
    w = int(shuffle_words(b).view("<u4")[0])
    for j in range(4):
        assert ((w >> (4 * j)) & 0xF, (w >> (4 * j + 16)) & 0xF) == (2 * j + 1, 2 * j + 2)


def test_tiled_hand_worked_position():
    # W13_SWIGLU, I = 128: tile t = 3 holds gate rows 24..31 (lanes n = 0..7)
    # and up rows 128+24..128+31 (n = 8..15). Lane l = 16*kq + n of group g
    # is the 16 bytes at plain byte offset 64g + 16kq of that row, each word
    # shuffled; its place is block b = 0, i = 3, at ((b*G + g)*8 + i)*1024 +
    # l*16 within the expert.
    E, N, K2 = 1, 256, 128
    G = 2
    plain = np.zeros((E, N, K2), np.uint8)
    row, g, kq, n = 128 + 24 + 5, 1, 2, 13            # up row of n = 13 in tile 3
    run = np.arange(1, 17, dtype=np.uint8)
    plain[0, row, 64 * g + 16 * kq: 64 * g + 16 * kq + 16] = run
    t = tiled_codes(plain, 0, 128).reshape(-1)
    pos = ((0 * G + g) * 8 + 3) * 1024 + (16 * kq + n) * 16
    assert np.array_equal(t[pos:pos + 16], shuffle_words(run))
    assert np.count_nonzero(t) == np.count_nonzero(shuffle_words(run))
