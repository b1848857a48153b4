"""Exact rational brute force used to pin the oracle on tiny inputs.

It shares nothing with the oracle: values are Python ``Fraction``s, binary32
rounding is done by integer arithmetic, and the E4M3 value set is enumerated
from its counting structure (codes 0x00..0x7E are the non-negative finite
values in increasing order) rather than decoded from bit fields.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

# ---- binary32 rounding ---------------------------------------------------


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(v: Fraction) -> int:
    f = v.numerator // v.denominator
    r = v - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def round_to_f32(v: Fraction, negative_zero: bool = False) -> float:
    """Nearest binary32 value (ties to even), subnormals kept, overflow to inf.
    ``negative_zero`` gives the sign of a zero result when v rounds to 0 from
    below."""
    if v == 0:
        return -0.0 if negative_zero else 0.0
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    e = _floor_log2(a)
    q = Fraction(2) ** (max(e, -126) - 23)
    n = _round_half_even(a / q)
    val = n * q
    if val >= Fraction(2) ** 128:
        return sign * float("inf")
    if n == 0:
        return -0.0 if sign < 0 else 0.0
    return sign * float(val)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bf16_to_fraction(bits: int) -> Fraction:
    x = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    return Fraction(x)


# ---- E4M3 value set by enumeration ----------------------------------------


def _e4m3_positive_values():
    vals = [Fraction(0)]
    vals += [Fraction(k, 2 ** 9) for k in range(1, 8)]  # subnormals
    e = -6
    while True:
        for m in range(8):
            v = Fraction(8 + m, 8) * Fraction(2) ** e
            if v > 448:
                return vals
            vals.append(v)
        e += 1


E4M3_POS = _e4m3_positive_values()  # index == code for codes 0x00..0x7E
assert len(E4M3_POS) == 127 and E4M3_POS[-1] == 448


def e4m3_value(code: int) -> Fraction:
    mag = code & 0x7F
    if mag == 0x7F:
        raise ValueError("NaN code")
    v = E4M3_POS[mag]
    return -v if code & 0x80 else v


def e4m3_nearest(y: float) -> int:
    """Brute-force nearest E4M3 code to the binary32 value y: search every
    finite code, break ties toward the even code, saturate beyond 448, keep
    the sign of y (including -0.0)."""
    neg = math.copysign(1.0, y) < 0
    a = abs(Fraction(y))
    if a >= 448:
        best = 126
    else:
        best, bestd = None, None
        for c, v in enumerate(E4M3_POS):
            d = abs(v - a)
            if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
                best, bestd = c, d
    return best | (0x80 if neg else 0)


# ---- tile quantization, exactly -----------------------------------------


def scale_of(amax: Fraction, pow2: bool) -> float:
    if amax == 0:
        return 1.0
    if not pow2:
        return round_to_f32(amax / 448)
    e = -200
    while 448 * Fraction(2) ** e < amax:
        e += 1
    return float(Fraction(2) ** e)


def quantize_values(xs, pow2: bool):
    """xs: list of (bits) BF16 in one tile -> (codes, scale)."""
    fr = [bf16_to_fraction(b) for b in xs]
    amax = max((abs(v) for v in fr), default=Fraction(0))
    s = scale_of(amax, pow2)
    codes = []
    for b, v in zip(xs, fr):
        neg = bool(b & 0x8000)
        y = round_to_f32(v / Fraction(s), negative_zero=neg)
        codes.append(e4m3_nearest(y))
    return codes, s


# ---- limited-precision accumulation, exactly -------------------------------


def _expo(t: Fraction) -> int:
    """E with 2^(E-1) <= |t| < 2^E, t != 0."""
    t = abs(t)
    e = t.numerator.bit_length() - t.denominator.bit_length()
    fl = e if t >= Fraction(2) ** e else e - 1
    return fl + 1


def limited_dot_exact(a, b, width: int, bits: int) -> float:
    """The limited-accumulation reading (each step aligns `width` products
    and the running sum to the largest term, truncates every term toward zero
    to a multiple of 2^(E - bits), and rounds the exact sum of the kept terms
    to binary32) evaluated with Python fractions and integer truncation.
    a, b: sequences of exact FP8 values (floats)."""
    acc = Fraction(0)
    for k0 in range(0, len(a), width):
        terms = [acc] + [Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a[k0:k0 + width], b[k0:k0 + width])]
        nz = [t for t in terms if t != 0]
        if not nz:
            acc = Fraction(0)
            continue
        lsb = Fraction(2) ** (max(_expo(t) for t in nz) - bits)
        s = sum(int(t / lsb) * lsb for t in terms)  # int() truncates toward zero
        acc = Fraction(round_to_f32(s))
    return float(acc)
