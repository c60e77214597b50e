"""Shared test helpers: device transfer of numpy inputs and the layer tolerance."""
import sys

import numpy as np

# Full-layer tolerance (floating point; MFMA accumulation order, the exp
# implementation and bf16 rounding points differ from the fp64 oracle):
#   max |gpu - ref| <= 2e-2 * max |ref|   and   sum |gpu - ref| / sum |ref| <= 5e-3
MAX_ABS_FRAC = 2e-2
MEAN_REL = 5e-3


def say(*a):
    """Name the case before a GPU step (unbuffered)."""
    print(*a, file=sys.stderr, flush=True)


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(a_u16):
    import torch
    return to_dev(np.ascontiguousarray(a_u16, dtype=np.uint16)).view(torch.bfloat16)


def to_np_u16(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(a_u16):
    return (np.asarray(a_u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def layer_errors(got_u16, ref_u16):
    g = bf16_to_f64(got_u16)
    r = bf16_to_f64(ref_u16)
    d = np.abs(g - r)
    max_ref = float(np.abs(r).max()) if r.size else 0.0
    max_err = float(d.max()) if d.size else 0.0
    mean_rel = float(d.sum() / max(np.abs(r).sum(), 1e-300)) if r.size else 0.0
    return max_err, max_ref, mean_rel


def assert_layer_close(got_u16, ref_u16, what=""):
    max_err, max_ref, mean_rel = layer_errors(got_u16, ref_u16)
    say(f"  {what}: max|d|={max_err:.3e} max|ref|={max_ref:.3e} ({max_err / max(max_ref, 1e-300):.2e}) "
        f"mean_rel={mean_rel:.2e}")
    assert max_err <= MAX_ABS_FRAC * max_ref, (what, max_err, max_ref)
    assert mean_rel <= MEAN_REL, (what, mean_rel)


def shuffle_words(b):
    """The tiled layout's word shuffle, from its definition in the C header:
    code c_j of a little-endian word (bits 4j..4j+3) moves to nibble j/2 for
    even j and to nibble 4 + (j-1)/2 for odd j. b: uint8 array, last axis a
    multiple of 4."""
    w = np.ascontiguousarray(b).view("<u4")
    out = np.zeros_like(w)
    for j in range(8):
        code = (w >> np.uint32(4 * j)) & np.uint32(0xF)
        dst = j // 2 if j % 2 == 0 else 4 + (j - 1) // 2
        out |= code << np.uint32(4 * dst)
    return out.view(np.uint8).reshape(b.shape)


def tiled_runs(wq, kind, inter):
    """The tiled layout's runs before any word shuffle (the tiled MXFP4 code
    layout as it is), from the definition in the C header:
    tiled[e][b][g][i][l] = plain[e][row(16*(8b+i), l%16)][64g + 16(l//16) : +16].
    kind 0 (W13_SWIGLU) pairs gate row 8t+n with up row I+8t+n in tile t."""
    wq = np.asarray(wq, np.uint8)
    E, N, K2 = wq.shape
    G = (2 * K2) // 128
    out = np.empty((E, N // 128, G, 8, 64, 16), np.uint8)
    for b in range(N // 128):
        for i in range(8):
            t = 8 * b + i
            for n in range(16):
                if kind == 0:
                    row = 8 * t + n if n < 8 else inter + 8 * t + n - 8
                else:
                    row = 16 * t + n
                for g in range(G):
                    for kq in range(4):
                        out[:, b, g, i, 16 * kq + n, :] = wq[:, row, 64 * g + 16 * kq: 64 * g + 16 * kq + 16]
    return out.reshape(E, N, K2)


def tiled_codes(wq, kind, inter):
    """The tiled int4 code layout from its definition in the C header: the
    runs of tiled_runs, each 4-byte word shuffled."""
    return shuffle_words(tiled_runs(wq, kind, inter)).reshape(np.asarray(wq).shape)
