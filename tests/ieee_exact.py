"""Exact-rational model of IEEE-754 round-to-nearest-even arithmetic.

A second, independent statement of the arithmetic the oracle is meant to do,
used to pin the oracle on tiny inputs: every operation is computed exactly
with fractions.Fraction and then rounded to the target format by the textbook
rule (the representable neighbour nearest the exact value, ties to the one
with an even last significand bit, overflow past the largest finite value plus
half an ulp to infinity).  Values are carried as Python floats, which hold
every binary32 and bfloat16 value exactly.
"""
from fractions import Fraction
import math

import numpy as np

# (significand bits p, minimum normal exponent, maximum exponent)
BINARY32 = (24, -126, 127)
BFLOAT16 = (8, -126, 127)


def round_to(q: Fraction, fmt) -> float:
    p, emin, emax = fmt
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** (emax + 1):
        return -math.inf if neg else math.inf
    f = float(v)
    return -f if neg else f


def add(a: float, b: float, fmt=BINARY32) -> float:
    if a == 0 and b == 0:
        return -0.0 if (math.copysign(1, a) < 0 and math.copysign(1, b) < 0) else 0.0
    s = Fraction(a) + Fraction(b)
    if s == 0:
        return 0.0
    return round_to(s, fmt)


def div(a: float, c: int, fmt=BINARY32) -> float:
    if a == 0:
        return a
    return round_to(Fraction(a) / c, fmt)


def bf16_bits_to_float(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


def float_to_bf16_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)


def float_to_f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def fold(values, bf16: bool, pre_div: bool, c: int) -> float:
    """Rank-order fp32 fold of one column's contributions, rounded at the end."""
    vs = []
    for x in values:
        v = x
        if pre_div:
            v = div(x, c)
            if bf16 and v != 0:
                v = round_to(Fraction(v), BFLOAT16)
        vs.append(v)
    acc = vs[0]
    for v in vs[1:]:
        acc = add(acc, v)
    if bf16 and acc != 0 and math.isfinite(acc):
        acc = round_to(Fraction(acc), BFLOAT16)
    return acc
