"""Exact-rational model of the slot-ordered combine (pure Python, fractions).

TEST INFRASTRUCTURE, part of the oracle. It pins the C oracle's binary32
multiply / fusedMultiplyAdd and its bf16 rounding without trusting any
floating-point unit: every product and sum is formed exactly as a Fraction and
rounded once, to nearest with ties to even, in the target format's full range
(subnormals included, no flush-to-zero).

Rule followed: the combine of the FlashInfer PR #7196 analysis ("CuTe DSL W4A16
MoE optimization and bitwise-exactness tests", section 1 `moe_finalize.py`):
the first slot is a plain fp32 multiply, each later slot an fp32 FMA in slot
order, FTZ removed; IEEE 754 fixes the sign of exact zero results.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

F32 = (24, -126, 128)   # significant bits, min normal exponent, overflow exponent
BF16 = (8, -126, 128)


def _is_neg(x: float) -> bool:
    return math.copysign(1.0, x) < 0


def round_to(x: Fraction, fmt=F32, neg_zero: bool = False) -> float:
    """Round an exact rational to the nearest value of `fmt` (ties to even).

    A zero rational returns -0.0 when neg_zero is set, else +0.0. Values whose
    rounded magnitude reaches 2^128 become infinity.
    """
    bits, emin, eover = fmt
    if x == 0:
        return -0.0 if neg_zero else 0.0
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, emin) - (bits - 1)          # exponent of one unit in the last place
    n = round(a / Fraction(2) ** q)         # Fraction.__round__: half to even
    v = Fraction(n) * Fraction(2) ** q
    if v >= Fraction(2) ** eover:
        r = math.inf
    else:
        r = float(v)                        # exact: v is representable
    if n == 0:
        return -0.0 if neg else 0.0
    return -r if neg else r


def mul_f32(a: float, b: float) -> float:
    """IEEE binary32 multiply, round to nearest even."""
    p = Fraction(a) * Fraction(b)
    return round_to(p, F32, neg_zero=(_is_neg(a) != _is_neg(b)))


def fma_f32(a: float, b: float, c: float) -> float:
    """IEEE binary32 fusedMultiplyAdd a*b + c with a single rounding."""
    p = Fraction(a) * Fraction(b)
    s = p + Fraction(c)
    if s == 0:
        pneg = _is_neg(a) != _is_neg(b)
        # exact zero: opposite-sign operands (or cancelling non-zeros) give +0
        # under round-to-nearest; two zeros of the same sign keep that sign.
        neg_zero = (p == 0 and c == 0 and pneg and _is_neg(c))
        return -0.0 if neg_zero else 0.0
    return round_to(s, F32)


def f32(x: float) -> float:
    """Value of x after a round trip through binary32 (x must already be binary32)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16_bits(x: float) -> int:
    """bf16 bit pattern of the RNE rounding of the (exact) value x."""
    if math.isnan(x):
        return 0xFFC0 if _is_neg(x) else 0x7FC0
    if math.isinf(x):
        return 0xFF80 if x < 0 else 0x7F80
    r = round_to(Fraction(x), BF16, neg_zero=_is_neg(x))
    u = struct.unpack("<I", struct.pack("<f", r))[0]
    return u >> 16


def combine(values, weights, present=None) -> float:
    """Ordered combine of one output element over the k slots.

    values / weights: sequences of binary32 numbers in slot order; present[j]
    False skips slot j (a slot routed to a non-local expert). Returns the
    binary32 accumulator (+0.0 when no slot is present).
    """
    acc = None
    for j, (v, w) in enumerate(zip(values, weights)):
        if present is not None and not present[j]:
            continue
        acc = mul_f32(v, w) if acc is None else fma_f32(v, w, acc)
    return 0.0 if acc is None else acc
