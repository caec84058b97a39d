"""Crafted RMSNorm rows whose mean square lies next to a binary32 rounding
midpoint, with the deciding part in squares 2^150 and 2^300 below the row's
largest.  Test inputs only: built with exact integer arithmetic from the
definition of the squares, independent of the oracle and the library.

Every square of a bf16 value a * 2^k (integer a < 256) is a^2 * 2^(2k + 266)
units of 2^-266.  Rows have 256 columns and a largest value 1.5 * 2^40,
whose square sits at 2^332 units; "levels" are 150-bit ranges counted down
from there: level 0 holds the squares of at least 2^182 units, level 1
those from 2^32, level 2 the rest.  The constructor picks the level-0
squares so that their sum is C m 2^84 - g, m a midpoint between two
adjacent binary32 numbers lo < hi near the mean square and 1 <= g <= 2^14,
then plants squares below level 0 that bring the total to just below,
exactly onto, or just above C m: the mean square rounds to lo, to the even
one of lo and hi, or to hi.
"""
from fractions import Fraction
from math import isqrt

import numpy as np

import workloads as W

C = 256
U0 = 182          # level 0 unit (exponent of 2^-266 units)
U1 = U0 - 150
U2 = U1 - 150
EPS = 1e-6

KINDS = {            # kind: expected rounding
    "tie": "even",
    "above_level1": "hi",
    "above_level2": "hi",
    "below": "lo",
    "level2_tie": "even",
    "level2_below": "lo",
    "level2_above": "hi",
}


def _four_squares(n):
    """n = a^2 + b^2 + c^2 + d^2 with 0 <= d <= c <= b <= a <= 127."""
    for a in range(min(127, isqrt(n)), -1, -1):
        r1 = n - a * a
        for b in range(min(a, isqrt(r1)), -1, -1):
            r2 = r1 - b * b
            for c in range(min(b, isqrt(r2)), -1, -1):
                r3 = r2 - c * c
                d = isqrt(r3)
                if d * d == r3 and d <= c:
                    return [a, b, c, d]
    raise ValueError(n)


def _units(a, k):
    return (a * a) << (2 * k + 266)


def _digits_as_squares(value, unit):
    """Values a * 2^k whose squares sum to value * 2^unit units exactly, for
    value a multiple of 2^14: base-2^14 digits from the second one up, each
    as four squares of integers below 128 (all at least 2^unit units, so in
    the level whose unit is `unit`)."""
    assert value % (1 << 14) == 0
    out = []
    j, v = 1, value >> 14
    while v:
        d = v & 0x3FFF
        k2 = unit + 14 * j - 266
        assert k2 % 2 == 0
        out += [(a, k2 // 2) for a in _four_squares(d) if a]
        v >>= 14
        j += 1
    return out


def _f32_parts(x: Fraction):
    """(m, q): x lies in [m 2^q, (m + 1) 2^q) with 2^q the last bit of the
    binary32 numbers there (normal range)."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    q = e - 23
    m = int(x / Fraction(2) ** q)
    return m, q


def mean_square_row(kind: str, seed: int):
    """(bf16 bits [C], lo, hi, expected) with lo < hi adjacent binary32
    numbers and expected the value the mean square must round to.  Seeds are
    stepped until lo and hi also give different inverse RMS values."""
    for s in range(seed, seed + 1000):
        rng = np.random.default_rng(s)
        vals = [(192, 33)]                                   # 1.5 * 2^40: the largest
        for _ in range(60):
            vals.append((int(rng.integers(128, 256)), int(rng.integers(13, 33))))
        a_base = sum(_units(a, k) for a, k in vals) >> U0
        assert sum(_units(a, k) for a, k in vals) % (1 << U0) == 0
        X = Fraction(a_base, C) * Fraction(2) ** (U0 - 266)  # mean of the level-0 part, real
        m, q = _f32_parts(X)
        if Fraction(2 * m + 1) * Fraction(2) ** (q - 1) <= X:
            m += 1                                           # the next midpoint up
        if m + 1 >= 1 << 24:
            continue                                         # keep lo and hi in one binade
        lo = np.float32(m * 2.0 ** q)
        hi = np.float32((m + 1) * 2.0 ** q)
        if not (np.float32(1) / np.sqrt(lo + np.float32(EPS)) != np.float32(1) / np.sqrt(hi + np.float32(EPS))):
            continue
        mid_units = Fraction(2 * m + 1) * Fraction(2) ** (q - 1 - (U0 - 266))
        assert mid_units.denominator == 1
        gap = C * int(mid_units) - a_base
        assert gap > 0
        g = (gap - 1) % (1 << 14) + 1
        vals += _digits_as_squares(gap - g, U0)
        # below level 0: squares of a * 2^-42 (a < 128) are a^2 units of 2^182
        # each, the rest by kind
        if kind in ("tie", "above_level1", "above_level2"):
            low = [(a, -42) for a in _four_squares(g) if a]
            if kind == "above_level1":
                low.append((1, -60))                          # 2^146 units: level 1
            elif kind == "above_level2":
                low.append((1, -120))                         # 2^26 units: level 2
        elif kind == "below":
            low = [(a, -42) for a in _four_squares(g - 1) if a] + [(1, -120)]
        else:
            # g - 1 at level 0 units, then 1 - 2^-136 of one such unit from
            # level 1 and 2^-136 (or less, or more) from level 2
            low = [(a, -42) for a in _four_squares(g - 1) if a]
            low += _digits_as_squares((1 << 150) - (1 << 14), U1)
            n = {"level2_tie": 4, "level2_below": 3, "level2_above": 4}[kind]
            low += [(1, -111)] * n                            # 2^162 units of 2^U2 each
            if kind == "level2_above":
                low.append((1, -125))
        vals += low
        assert len(vals) <= C
        row = np.zeros(C, np.float32)
        for i, (a, k) in enumerate(vals):
            row[i] = np.float32(a * 2.0 ** k) * (1 if rng.random() < 0.5 else -1)
        row = row[rng.permutation(C)]
        bits = W.f32_to_bf16_bits(row)
        assert np.array_equal(W.bf16_bits_to_f32(bits), row)  # every value exact in bf16
        exp = KINDS[kind]
        want = {"lo": lo, "hi": hi, "even": lo if (int(lo.view(np.uint32)) & 1) == 0 else hi}[exp]
        return bits, lo, hi, np.float32(want)
    raise RuntimeError("no seed separates the inverse RMS of lo and hi")


def exact_mean_square(bits) -> Fraction:
    """sum x^2 / C as a Fraction, straight from the float values."""
    return sum(Fraction(float(v)) ** 2 for v in W.bf16_bits_to_f32(bits)) / len(bits)
