"""Exact rational arithmetic helpers for pinning the oracle (tests only).

round_fp32 rounds an exact rational to the nearest IEEE binary32 value with
ties to even (subnormals included), straight from the format definition, so
fp32 operation sequences can be re-derived without floating-point hardware.
"""
from fractions import Fraction

import numpy as np

_TWO = Fraction(2)


def frac(x) -> Fraction:
    return Fraction(float(x))


def round_fp32(q: Fraction) -> np.float32:
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = _TWO ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= _TWO ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))
    return -out if neg else out


def fmaf_exact(a, b, c) -> np.float32:
    return round_fp32(frac(a) * frac(b) + frac(c))


def sub_exact(a, b) -> np.float32:
    return round_fp32(frac(a) - frac(b))


def dist8_exact_chain(r, c) -> np.float32:
    """The fp32 operation sequence e = r_k - c_k; acc = fma(e, e, acc), k = 0..7,
    evaluated with exact rationals and one rounding per operation."""
    acc = np.float32(0.0)
    for k in range(8):
        e = sub_exact(r[k], c[k])
        acc = fmaf_exact(e, e, acc)
    return acc


def dist8_real(r, c) -> Fraction:
    """The true squared distance of the fp32 values (no rounding at all)."""
    return sum((frac(r[k]) - frac(c[k])) ** 2 for k in range(8))
