"""Pins of the oracle's and the generator's bf16 rounding (no GPU).

bf16 keeps 8 significant bits and binary32's exponent range; rounding is to
nearest, ties to even, through the subnormal range and to infinity at 2^128.
The exact-rational rounding in oracle/exact.py is the reference.
"""
import math
from fractions import Fraction

import numpy as np

import oracle
from oracle import exact
from w4a16_grouped_gemm_amd.inputs import bf16_bits, bf16_values


def test_double_to_bf16_edges():
    cases = [0.0, -0.0, 1.0, -1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 1.0 + 2**-9 + 2**-40,
             2**-126, 2**-127, 2**-133, 2**-134, 3 * 2**-135, 2**-134 + 2**-160,
             (2 - 2**-7) * 2**127, (2 - 2**-8) * 2**127, (2 - 2**-9) * 2**127, 2.0**128, -2.0**130,
             math.inf, -math.inf, 1e-40, -3.1e-39, 0.1, 1 / 3]
    for d in cases:
        want = exact.bf16_bits(d)
        assert oracle.bf16_from_double(d) == want, d


def test_double_to_bf16_random():
    rng = np.random.default_rng(11)
    ds = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-45, 40, 3000),
                         (rng.integers(1, 1 << 20, 2000) * 2.0 ** -rng.integers(120, 150, 2000))])
    for d in ds:
        assert oracle.bf16_from_double(float(d)) == exact.bf16_bits(float(d)), d


def test_ties_round_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even mantissa -> 1.0
    assert oracle.bf16_from_double(1 + 2**-8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: -> 1+2^-6 (even)
    assert oracle.bf16_from_double(1 + 3 * 2**-8) == 0x3F82


def test_generator_f32_to_bf16():
    rng = np.random.default_rng(12)
    f = np.concatenate([rng.standard_normal(4000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.array([0.0, -0.0, 1 + 2**-8, 3e38], np.float32)])
    got = bf16_bits(f)
    for v, g in zip(f, got):
        assert int(g) == exact.bf16_bits(float(v))
    assert np.array_equal(bf16_bits(bf16_values(got)), got)
