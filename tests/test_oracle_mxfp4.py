"""Pins of the W4A4 (MXFP4) oracle, against things other than itself.

- The E2M1 decode of all 16 codes and hand-derived quantized blocks
  (tests/golden/mxfp4_cases.json: ties, saturation, zero block, subnormal
  maximum, signed zero).
- Quantization properties that pin it without retyping it: every element's
  code is a nearest point of the block's scaled grid (checked against all 16
  codes), ties land on even codes, the scale puts the block maximum in
  [4, 8) (unless clamped), and blocks built from representable values
  round-trip exactly.
- The grouped GEMM: exact against numpy's float64 matmul of the dequantised
  operands (small E2M1 products and power-of-two scales keep every sum
  exact); one-hot activations read weight columns back; gate/up split.
- The layer: the permuted path equals the per-token brute force bit for bit,
  and one expert with all-local slots reduces to a dense numpy FFN.
"""
import json
import os

import numpy as np
import pytest

import oracle
from w4a16_grouped_gemm_amd.inputs import bf16_bits, bf16_values, make_mxfp4_layer_inputs, pack_int4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_cases.json")
E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)])


def _unpack_codes(codes):
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def _dequant(codes, scales):
    c = _unpack_codes(codes)
    v = E2M1[c]
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    return v * s


def _pack_codes(c):
    c = np.asarray(c, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_e2m1_decode_table():
    g = json.load(open(GOLDEN))
    for row in g["e2m1"]:
        v = oracle.e2m1_value(row["code"])
        assert v == row["value"] and np.signbit(v) == bool(row["sign"]), row
        assert row["code"] == row["sign"] * 8 + row["exp"] * 2 + row["man"]
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(0) == 2.0 ** -127 and oracle.e8m0_value(130) == 8.0


def test_quantize_golden_blocks():
    g = json.load(open(GOLDEN))
    for b in g["blocks"]:
        if "values_bf16_bits" in b:
            head = np.array(b["values_bf16_bits"], np.uint16)
        else:
            head = bf16_bits(np.array(b["values"], np.float32))
        blk = np.full(32, bf16_bits(np.float32(b["fill"])), np.uint16)
        blk[: len(head)] = head
        codes, scales = oracle.mx_quantize(blk[None, :])
        c = _unpack_codes(codes)[0]
        assert scales[0, 0] == b["scale"], b["what"]
        n = len(head)
        assert list(c[:n]) == b["codes"], (b["what"], list(c[:n]))
        assert np.all(c[n:] == b["fill_code"]), b["what"]


def _random_blocks(rng, n):
    # N(0,1) scaled per block by 2^U[-20, 20], plus values placed exactly on
    # grid midpoints, so ties occur
    x = rng.standard_normal((n, 32)) * np.ldexp(1.0, rng.integers(-20, 21, size=(n, 1)))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for i in range(0, n, 3):
        amax_exp = rng.integers(-10, 10)
        x[i, 0] = 4.0 * 2.0 ** amax_exp                       # block max on the grid: X = 2^amax_exp
        x[i, 1:8] = mids * 2.0 ** amax_exp * rng.choice([-1, 1], size=7)
    return bf16_bits(x.astype(np.float32))


def test_quantize_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(3)
    xb = _random_blocks(rng, 600)
    codes, scales = oracle.mx_quantize(xb)
    x = bf16_values(xb).astype(np.float64)
    c = _unpack_codes(codes)
    X = np.ldexp(1.0, scales[:, 0].astype(np.int64) - 127)[:, None]
    amax = np.abs(x).max(axis=1)
    # the scale puts the block maximum in [4, 8) on the E2M1 scale
    ok = amax > 0
    assert np.all(amax[ok] / X[ok, 0] >= 4.0) and np.all(amax[ok] / X[ok, 0] < 8.0)
    # each code is a nearest point of X * {E2M1} (saturating at 6); ties even
    p = x / X
    got = E2M1[c]
    dist = np.abs(np.abs(p)[..., None] - np.abs(E2M1[:8])[None, None, :])
    best = dist.min(axis=-1)
    mine = np.abs(np.abs(p) - np.abs(got))
    sat = np.abs(p) > 6.0
    assert np.all(np.where(sat, np.abs(got) == 6.0, mine == best))
    tie = (np.sum(dist == best[..., None], axis=-1) == 2) & ~sat
    assert tie.sum() > 100
    assert np.all((c[tie] & 1) == 0)
    # the sign of the input is kept (codes 8..15 for negative inputs and -0)
    assert np.all((c >= 8) == np.signbit(x))


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(4)
    n = 200
    c = rng.integers(0, 16, size=(n, 32)).astype(np.uint8)
    c[:, 0] = rng.choice([6, 7, 14, 15], size=n)               # a +-4 or +-6 fixes the scale
    s = rng.integers(100, 150, size=(n, 1)).astype(np.uint8)
    x = _dequant(_pack_codes(c), s)
    codes, scales = oracle.mx_quantize(bf16_bits(x.astype(np.float32)))
    assert np.array_equal(scales, s)
    assert np.array_equal(_unpack_codes(codes), c)


def _mx_weights(rng, E, N, K, smin=120, smax=124):
    codes = _pack_codes(rng.integers(0, 16, size=(E, N, K)).astype(np.uint8))
    scales = rng.integers(smin, smax + 1, size=(E, N, K // 32)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("kind", [oracle.RAW, oracle.W2])
def test_gemm_exact_against_numpy(kind):
    rng = np.random.default_rng(11 + kind)
    E, N, K = 3, 64, 256
    wq, ws = _mx_weights(rng, E, N, K)
    counts = np.array([5, 0, 9])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    aq, as_ = _mx_weights(rng, 1, R, K, 124, 130)
    aq, as_ = aq[0], as_[0]
    got = oracle.grouped_gemm_mxfp4(kind, aq, as_, offsets, wq, ws, rows=R, out_f32=True)
    A = _dequant(aq, as_)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        want = A[r0:r1] @ _dequant(wq[e], ws[e]).T
        assert np.array_equal(got[r0:r1].astype(np.float64), want)


def test_gemm_one_hot_and_gather():
    rng = np.random.default_rng(12)
    E, N, K = 2, 32, 128
    wq, ws = _mx_weights(rng, E, N, K, 110, 140)
    W = _dequant(wq, ws)
    ks = rng.integers(0, K, size=6)
    c = np.zeros((6, K), np.uint8)
    c[np.arange(6), ks] = 2                                      # E2M1 1.0
    aq = _pack_codes(c)
    as_ = np.full((6, K // 32), 127, np.uint8)
    idx = np.array([10, 2, 7, 1, 9, 4], np.int32)                # gather: a row = idx // 2 (distinct)
    offsets = np.array([0, 4, 6], np.int32)
    src = np.zeros((6, K // 2), np.uint8)
    ssrc = np.zeros((6, K // 32), np.uint8)
    src[idx // 2] = aq
    ssrc[idx // 2] = as_
    got = oracle.grouped_gemm_mxfp4(oracle.RAW, src, ssrc, offsets, wq, ws, rows=6, a_row_index=idx, top_k=2,
                                    out_f32=True)
    for r in range(6):
        e = 0 if r < 4 else 1
        assert np.array_equal(got[r].astype(np.float64), W[e][:, ks[r]]), r


def test_gemm_swiglu_split():
    # rows [0, I) are the gate, [I, 2I) the up projection
    rng = np.random.default_rng(13)
    I, K = 32, 64
    wq, ws = _mx_weights(rng, 1, 2 * I, K)
    aq, as_ = _mx_weights(rng, 1, 3, K, 125, 128)
    offsets = np.array([0, 3], np.int32)
    h = oracle.grouped_gemm_mxfp4(oracle.W13_SWIGLU, aq[0], as_[0], offsets, wq, ws, rows=3)
    raw = oracle.grouped_gemm_mxfp4(oracle.RAW, aq[0], as_[0], offsets, wq, ws, rows=3, out_f32=True)
    g, u = raw[:, :I].astype(np.float64), raw[:, I:].astype(np.float64)
    want = g / (1.0 + np.exp(-g)) * u
    assert np.all(np.abs(bf16_values(h) - want) <= 2.0 ** -8 * np.abs(want) + 1e-30)


@pytest.mark.parametrize("wl,T", [("tiny", 16), ("tiny", 5), ("ep_shard_decode", 2)])
def test_layer_equals_bruteforce(wl, T):
    inp = make_mxfp4_layer_inputs(wl, T)
    w = inp.workload
    r = oracle.layer_w4a4(inp.x, inp.logits, inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s, top_k=w.top_k,
                          expert_begin=w.expert_begin)
    bf = oracle.layer_w4a4_bruteforce(inp.x, r["topk_ids"], r["topk_w"], inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s,
                                      expert_begin=w.expert_begin)
    assert np.array_equal(r["out"], bf)


def test_layer_one_expert_is_a_dense_ffn():
    # E = 1, k = 1: weight 1 on every token, so the layer is the dense W4A4
    # FFN of each token, written here with numpy on dequantised operands
    from w4a16_grouped_gemm_amd.inputs import Workload
    wl = Workload("one_expert", 30, 1, 1, 0, 1, 128, 128, (6,))
    inp = make_mxfp4_layer_inputs(wl, 6)
    r = oracle.layer_w4a4(inp.x, inp.logits, inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s, top_k=1)
    xq, xs = oracle.mx_quantize(inp.x)
    A = _dequant(xq, xs)
    W13 = _dequant(inp.w13_q[0], inp.w13_s[0])
    gu = A @ W13.T
    g, u = gu[:, :128], gu[:, 128:]
    h = bf16_bits((g / (1.0 + np.exp(-g)) * u).astype(np.float32))
    # h computed in fp64 then rounded once in the oracle; compare after its own rounding
    assert np.all(np.abs(bf16_values(h) - bf16_values(r["h"])) <= 2.0 ** -7 * np.abs(bf16_values(r["h"])))
    hq, hs = oracle.mx_quantize(r["h"])
    y = _dequant(hq, hs) @ _dequant(inp.w2_q[0], inp.w2_s[0]).T
    assert np.all(np.abs(bf16_values(r["y"]) - y) <= 2.0 ** -8 * np.abs(y) + 1e-30)
    assert np.array_equal(r["out"], r["y"])                  # weight 1: out = RNE(y * 1)
