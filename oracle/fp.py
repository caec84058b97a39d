"""Exact binary floating-point helpers of the oracle (integer arithmetic only).

TEST INFRASTRUCTURE.  Part of the CPU oracle; see ``oracle/__init__.py``.

Everything here decides a rounding with integers: no float division, no float
subtraction of non-exact operands.  The formats are IEEE 754 binary32 and
bfloat16 (the upper half of binary32) and the OCP 8-bit floating point format
E4M3FN (bias 7, largest finite value 448, no infinities, one NaN pattern per
sign).  These formats are outside the pages, which only name the precisions
(the GVCLab research log of 2026-09-02, section 5.5 table, SageAttention2
row: INT4 QK^T with FP8/FP16 PV).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32_MIN_EXP = -149          # exponent of the smallest binary32 subnormal
F32_MANT_BITS = 24


# ---------------------------------------------------------------------------
# decompositions
# ---------------------------------------------------------------------------

def bf16_parts(bits: np.ndarray):
    """bf16 bit patterns -> (neg, m, e) with value = (-1)^neg * m * 2^e exactly.

    m is the integer significand (0 <= m < 256, hidden bit included for
    normals), e the exponent of its last bit."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    neg = (b >> 15) & 1
    E = (b >> 7) & 0xFF
    F = b & 0x7F
    if np.any(E == 0xFF):
        raise ValueError("bf16 input holds an Inf or NaN")
    m = np.where(E > 0, F | 0x80, F)
    e = np.maximum(E, 1) - 134
    return neg, m, e


def f32_parts(x: np.ndarray):
    """float32 values -> (neg, m, e), value = (-1)^neg * m * 2^e, with m
    normalised to [2^23, 2^24) for nonzero values (subnormals shifted up) and
    m = 0 for zeros."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    neg = (u >> 31) & 1
    E = (u >> 23) & 0xFF
    F = u & 0x7FFFFF
    if np.any(E == 0xFF):
        raise ValueError("float32 input holds an Inf or NaN")
    m = np.where(E > 0, F | 0x800000, F)
    e = np.maximum(E, 1) - 150
    # normalise subnormals
    for _ in range(24):
        low = (m > 0) & (m < (1 << 23))
        if not low.any():
            break
        m = np.where(low, m << 1, m)
        e = np.where(low, e - 1, e)
    return neg, m, e


def _bit_length(n: np.ndarray) -> np.ndarray:
    """Bit length of non-negative int64 values below 2^62 (0 -> 0)."""
    n = np.asarray(n, dtype=np.int64)
    bl = np.zeros(n.shape, np.int64)
    for s in (32, 16, 8, 4, 2, 1):
        big = (n >> bl) >= (np.int64(1) << s)
        bl = np.where(big, bl + s, bl)
    return np.where(n > 0, bl + 1, 0)


def _assemble_f32(neg, mant, lsb_exp) -> np.ndarray:
    """(-1)^neg * mant * 2^lsb_exp -> float32, where the value is known to be a
    binary32 number (mant < 2^25 and lsb_exp >= -149) or overflows."""
    mant = np.asarray(mant, np.int64)
    lsb_exp = np.asarray(lsb_exp, np.int64)
    val = np.ldexp(mant.astype(np.float64), lsb_exp.astype(np.int32))   # exact in float64
    with np.errstate(over="ignore"):
        out = val.astype(np.float32)   # exact: val is representable (or overflows to inf)
    return np.where(np.asarray(neg) == 1, -out, out).astype(np.float32)


def round_scaled_int_to_f32(neg, n, e, sticky=None) -> np.ndarray:
    """Round (-1)^neg * (n + tail) * 2^e to binary32, nearest-even.

    n: non-negative int64 below 2^62; tail is an extra fraction in (0, 1) of the
    last unit of n, present where ``sticky`` is true (it only breaks ties).
    Subnormal results and overflow to infinity are handled."""
    n = np.asarray(n, np.int64)
    e = np.broadcast_to(np.asarray(e, np.int64), n.shape)
    neg = np.broadcast_to(np.asarray(neg, np.int64), n.shape)
    sticky = np.zeros(n.shape, bool) if sticky is None else np.broadcast_to(sticky, n.shape)
    nb = _bit_length(n)
    lsb = np.maximum(e + nb - F32_MANT_BITS, F32_MIN_EXP)       # exponent of the result's last bit
    sh = np.maximum(lsb - e, 0)                                  # bits dropped from n
    sh_c = np.minimum(sh, 62)
    mant = np.where(sh >= 63, 0, n >> sh_c)
    rem = np.where(sh >= 63, n, n - (mant << sh_c))
    half = np.where(sh >= 1, np.int64(1) << np.maximum(sh_c - 1, 0), 0)
    # sh >= 63 only happens deep below the subnormal range, where n < 2^62 is
    # below half a unit: no rounding up there.
    up = ((sh >= 1) & (sh <= 62)
          & ((rem > half) | ((rem == half) & (sticky | ((mant & 1) == 1)))))
    mant = mant + up.astype(np.int64)
    lsb = np.where(sh > 0, lsb, e)
    zero = (n == 0)
    mant = np.where(zero, 0, mant)
    return _assemble_f32(neg, mant, np.where(zero, 0, lsb))


def rational_to_f32(num: int, den: int) -> np.float32:
    """Round the exact rational num/den (den > 0) to binary32, nearest-even."""
    if den <= 0:
        raise ValueError("den must be positive")
    if num == 0:
        return np.float32(0.0)
    neg = num < 0
    n = abs(num)
    # e: 2^e <= n/den < 2^(e+1)
    e = n.bit_length() - den.bit_length()
    if (n << max(0, -e)) < (den << max(0, e)):
        e -= 1
    lsb = max(e - (F32_MANT_BITS - 1), F32_MIN_EXP)
    # q = n / (den * 2^lsb)
    if lsb >= 0:
        qn, qd = n, den << lsb
    else:
        qn, qd = n << (-lsb), den
    q, r = divmod(qn, qd)
    if 2 * r > qd or (2 * r == qd and (q & 1)):
        q += 1
    if q * 2.0 ** lsb >= 2.0 ** 128:
        return np.float32(-np.inf if neg else np.inf)
    v = np.float32(np.ldexp(float(q), lsb))
    return np.float32(-v) if neg else v


def f32_to_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


# ---------------------------------------------------------------------------
# binary32 operations on exact operands
# ---------------------------------------------------------------------------

def div_f32(x: np.ndarray, s) -> np.ndarray:
    """Correctly rounded binary32 quotient fl32(x / s), nearest-even.

    x: float32 array, s: float32 scalar or array (broadcast), s != 0, finite.
    Long division of the 24-bit significands with a remainder for the sticky
    bit; no floating-point division is used."""
    x = np.asarray(x, np.float32)
    s = np.broadcast_to(np.asarray(s, np.float32), x.shape)
    nx, mx, ex = f32_parts(x)
    ns, ms, es = f32_parts(s)
    if np.any(ms == 0):
        raise ZeroDivisionError("div_f32 by zero")
    num = mx << 26                                # < 2^50
    q = num // ms                                 # in (2^25, 2^27) for nonzero x
    r = num - q * ms
    out = round_scaled_int_to_f32(nx ^ ns, q, ex - es - 26, sticky=(r != 0))
    return np.where(mx == 0, np.where((nx ^ ns) == 1, np.float32(-0.0), np.float32(0.0)),
                    out).astype(np.float32)


def sub_bf16_f32(k_bits: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """fl32(K - mu): K given as bf16 bits, mu float32 (broadcast); exact
    difference, one nearest-even rounding to binary32 (subnormals kept)."""
    nk, mk, ek = bf16_parts(k_bits)
    mu = np.broadcast_to(np.asarray(mu, np.float32), mk.shape)
    nm, mm, em = f32_parts(mu)
    e0 = np.minimum(np.where(mk > 0, ek, em), np.where(mm > 0, em, ek))
    shk = ek - e0
    shm = em - e0
    fast = ((mk == 0) | (shk + 8 <= 61)) & ((mm == 0) | (shm + 24 <= 61))
    shk_c = np.where(fast & (mk > 0), shk, 0)
    shm_c = np.where(fast & (mm > 0), shm, 0)
    a = np.where(nk == 1, -1, 1) * (mk << shk_c)
    b = np.where(nm == 1, -1, 1) * (mm << shm_c)
    diff = a - b
    out = round_scaled_int_to_f32((diff < 0).astype(np.int64), np.abs(diff), e0)
    # exact zero difference is +0 in round-to-nearest
    out = np.where(diff == 0, np.float32(0.0), out).astype(np.float32)
    if not fast.all():
        idx = np.nonzero(~fast)
        kf = (np.asarray(k_bits, np.uint16)[idx].astype(np.uint32) << 16).view(np.float32)
        for j, (kv, mv) in enumerate(zip(kf, mu[idx])):
            fr = Fraction(float(kv)) - Fraction(float(mv))
            out[tuple(ix[j] for ix in idx)] = rational_to_f32(fr.numerator, fr.denominator)
    return out


def rne_to_int(q: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest integer, ties to even (exact)."""
    n, m, e = f32_parts(q)
    sh = np.clip(-e, 0, 62)
    k = np.where(e >= 0, m << np.clip(e, 0, 8), m >> sh)   # |q| here stays below 2^32
    rem = np.where(e >= 0, 0, m - (k << sh))
    half = np.where(sh >= 1, np.int64(1) << np.maximum(sh - 1, 0), 0)
    up = (e < 0) & ((rem > half) | ((rem == half) & ((k & 1) == 1)))
    k = k + up.astype(np.int64)
    return np.where(n == 1, -k, k)


def f32_to_bf16(y: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns, nearest-even (exact, integers only).

    bf16 keeps the upper 16 bits of binary32; the lower 16 decide the
    rounding: above half rounds up, exactly half rounds to the even upper
    part.  A carry into the exponent is the correct next binade (the largest
    finite values round to infinity).  NaN maps to the quiet NaN with the same
    sign and upper payload bits; infinities stay."""
    u = np.ascontiguousarray(y, dtype=np.float32).view(np.uint32).astype(np.int64)
    hi = u >> 16
    lo = u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = hi + up.astype(np.int64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    out = np.where(nan, hi | 0x40, out)
    return out.astype(np.uint16)


# ---------------------------------------------------------------------------
# OCP E4M3FN
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """binary32 -> OCP E4M3FN code (uint8), nearest-even, saturating to +-448.

    Quantum is 2^(k-3) in binade [2^k, 2^(k+1)) for k >= -6 and 2^-9 below
    (subnormals).  The sign bit follows the sign of y (also for zero)."""
    n, m, e = f32_parts(y)
    k = e + 23                                           # binade of |y| (m normalised)
    qe = np.maximum(k - 3, -9)                           # quantum exponent
    sh = qe - e                                          # >= 20 for normalised m
    sh_c = np.clip(sh, 0, 62)
    c = np.where(sh >= 63, 0, m >> sh_c)
    rem = m - (c << sh_c)
    half = np.int64(1) << np.maximum(sh_c - 1, 0)
    up = (rem > half) | ((rem == half) & ((c & 1) == 1))
    c = c + up.astype(np.int64)                          # |y| ~= c * 2^qe, c <= 16
    c = np.where(m == 0, 0, c)
    # normalise: c in [8, 16] for normal binades
    bump = c >= 16
    c = np.where(bump, c >> 1, c)
    qe = np.where(bump, qe + 1, qe)
    sub = (qe == -9) & (c < 8)
    E = np.where(sub, 0, qe + 3 + 7)
    mant = np.where(sub, c, c - 8)
    code = (E << 3) | mant
    sat = (E > 15) | ((E == 15) & (mant == 7))
    code = np.where(sat, 0x7E, code)
    return (code | (n << 7)).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """OCP E4M3FN code -> float64 value (NaN patterns 0x7F/0xFF -> nan)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    neg = (c >> 7) & 1
    E = (c >> 3) & 0xF
    F = c & 7
    mag = np.where(E == 0, np.ldexp(F.astype(np.float64), -9),
                   np.ldexp((8 + F).astype(np.float64), (E - 10).astype(np.int32)))
    mag = np.where((E == 15) & (F == 7), np.nan, mag)
    return np.where(neg == 1, -mag, mag)
