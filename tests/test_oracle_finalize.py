"""Pins of the oracle's ordered combine (no GPU).

The C oracle's binary32 multiply / fmaf and its bf16 rounding are checked
against (a) hand-derived IEEE results in tests/golden/finalize_cases.json and
(b) the exact-rational model in oracle/exact.py, which forms every product and
sum as a Fraction and rounds once. Rule: FlashInfer PR #7196 analysis, section
1 `moe_finalize.py` (fp32 multiply for slot 0, then fp32 FMA in slot order,
no FTZ).
"""
import json
import os
import struct

import numpy as np
import pytest

import oracle
from oracle import exact

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f32_from_hex(h):
    return struct.unpack("<f", struct.pack("<I", int(h, 16)))[0]


def bits32(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def run_c_finalize(values, weights, present=None, out_f32=True):
    """One token, H=1: feed the C oracle a [k,1] y and an identity inv_perm."""
    k = len(values)
    y = np.array(values, np.float32).reshape(k, 1)
    w = np.array(weights, np.float32).reshape(1, k)
    inv = np.arange(k, dtype=np.int32).reshape(1, k)
    if present is not None:
        inv = np.where(np.array(present)[None, :], inv, -1).astype(np.int32)
    out = oracle.finalize(y, w, inv, out_f32=out_f32)
    return out[0, 0]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "finalize_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_golden_cases(case):
    ys = [f32_from_hex(v) for v in case["y"]]
    ws = [f32_from_hex(v) for v in case["w"]]
    want = int(case["out"], 16)
    assert bits32(exact.combine(ys, ws)) == want
    assert bits32(float(run_c_finalize(ys, ws))) == want
    # bf16 output is the RNE rounding of the fp32 accumulator
    got16 = int(run_c_finalize(ys, ws, out_f32=False))
    assert got16 == exact.bf16_bits(f32_from_hex(case["out"]))


def _stress_values(rng, n):
    kind = rng.random(n)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    v = np.where(kind < 0.5, rng.standard_normal(n),
                 np.where(kind < 0.65, sign * 0.0,
                          np.where(kind < 0.8, sign * 10.0 ** rng.uniform(-45, -38, n),
                                   sign * 2.0 ** rng.integers(-80, -60, n))))
    return v.astype(np.float32)


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_random_against_exact_rationals(k):
    rng = np.random.default_rng(100 + k)
    T, H = 48, 24
    y = _stress_values(rng, T * k * H).reshape(T * k, H)
    w = rng.standard_normal((T, k)).astype(np.float32)
    w[rng.random((T, k)) < 0.15] = 0.0
    w[rng.random((T, k)) < 0.05] = -0.0
    # cancellation rows: slot 1 = -slot 0 so FMA and mul+add differ
    y[1::k] = -y[0::k] if k > 1 else y[1::k]
    inv = np.arange(T * k, dtype=np.int32).reshape(T, k)
    absent = rng.random((T, k)) < 0.2
    inv = np.where(absent, -1, inv).astype(np.int32)
    got32 = oracle.finalize(y, w, inv, out_f32=True)
    got16 = oracle.finalize(y, w, inv, out_f32=False)
    for t in range(T):
        for c in range(H):
            vals = [float(y[t * k + j, c]) for j in range(k)]
            ref = exact.combine(vals, [float(x) for x in w[t]], present=[not a for a in absent[t]])
            assert bits32(float(got32[t, c])) == bits32(ref), (t, c)
            assert int(got16[t, c]) == exact.bf16_bits(ref), (t, c)


def test_k1_is_one_correctly_rounded_multiply():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((500, 1)).astype(np.float32)
    w = rng.standard_normal((500, 1)).astype(np.float32)
    inv = np.zeros((1, 1), np.int32)
    for i in range(500):
        got = oracle.finalize(y[i:i + 1], w[i:i + 1], inv, out_f32=True)[0, 0]
        prod = np.float32(np.float64(y[i, 0]) * np.float64(w[i, 0]))  # exact double, one rounding
        assert bits32(float(got)) == bits32(float(prod))


def test_no_present_slot_gives_positive_zero():
    out = oracle.finalize(np.ones((2, 4), np.float32), np.ones((1, 2), np.float32),
                          np.full((1, 2), -1, np.int32), out_f32=True)
    assert all(bits32(float(v)) == 0 for v in out[0])


def test_bf16_input_path_matches_fp32_of_same_values():
    rng = np.random.default_rng(3)
    from w4a16_grouped_gemm_amd.inputs import bf16_bits, bf16_values
    yb = bf16_bits(rng.standard_normal((6, 32)).astype(np.float32))
    w = rng.standard_normal((2, 3)).astype(np.float32)
    inv = np.arange(6, dtype=np.int32).reshape(2, 3)
    a = oracle.finalize(yb, w, inv, out_f32=True)
    b = oracle.finalize(bf16_values(yb), w, inv, out_f32=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
