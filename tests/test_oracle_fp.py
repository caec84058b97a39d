"""Pins of the oracle's exact floating-point helpers.

Each helper is checked against something other than itself: the host CPU's
IEEE 754 binary32 arithmetic (numpy float32 division, subtraction, rint),
torch's CPU float8_e4m3fn conversion, exact rational arithmetic with
``fractions.Fraction`` (the definition of "nearest, ties to even"), and the
value table of the OCP 8-bit floating point specification (E4M3FN).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp
import workloads as W


def _nearest_check(x_frac: Fraction, r: np.float32):
    """r is the binary32 value nearest to x (ties to the even significand)."""
    r = np.float32(r)
    lo = np.nextafter(r, np.float32(-np.inf), dtype=np.float32)
    hi = np.nextafter(r, np.float32(np.inf), dtype=np.float32)
    dr = abs(Fraction(float(r)) - x_frac)
    for nb in (lo, hi):
        if not np.isfinite(nb):
            continue
        dn = abs(Fraction(float(nb)) - x_frac)
        assert dr <= dn, (x_frac, r, nb)
        if dr == dn:  # tie: r must have an even significand
            assert int(np.float32(r).view(np.uint32)) & 1 == 0, (x_frac, r)


def test_rational_to_f32_is_nearest():
    rng = np.random.default_rng(11)
    for _ in range(3000):
        num = int(rng.integers(-2**62, 2**62))
        den = int(rng.integers(1, 2**40))
        sh = int(rng.integers(-170, 120))
        frac = Fraction(num, den) * (Fraction(2) ** sh)
        r = fp.rational_to_f32(frac.numerator, frac.denominator)
        if np.isinf(r):
            assert abs(frac) >= Fraction(2) ** 128 - Fraction(2) ** 103
            continue
        _nearest_check(frac, r)


def test_rational_to_f32_ties_and_subnormals():
    # exact ties between consecutive binary32 values round to even
    one = Fraction(1)
    ulp = Fraction(2) ** -23
    assert fp.rational_to_f32(*(one + ulp / 2).as_integer_ratio()) == np.float32(1.0)
    r = fp.rational_to_f32(*(one + ulp + ulp / 2).as_integer_ratio())
    assert r == np.float32(1.0 + 2 * 2.0 ** -23)
    # smallest subnormal and half of it (tie -> 0, even)
    assert fp.rational_to_f32(1, 2**149) == np.float32(2.0 ** -149)
    assert fp.rational_to_f32(1, 2**150) == np.float32(0.0)
    assert fp.rational_to_f32(3, 2**150) == np.float32(2.0 ** -148)


def _wide_f32(rng, n, lo=-140, hi=60):
    x = rng.standard_normal(n) * np.exp2(rng.uniform(lo, hi, n))
    return x.astype(np.float32)


def test_div_f32_matches_ieee_division():
    rng = np.random.default_rng(5)
    x = _wide_f32(rng, 400_000)
    s = np.abs(_wide_f32(rng, 400_000, -120, 40))
    s[s == 0] = np.float32(1.0)
    got = fp.div_f32(x, s)
    ref = x / s                         # host binary32 division (IEEE, correctly rounded)
    ok = np.isfinite(ref)
    assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


def test_div_f32_quantizer_operands_exhaustive_bf16():
    # every finite bf16 pattern divided by scales of the a/127 form
    bits = np.arange(65536, dtype=np.uint16)
    x = W.bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    for a in (np.float32(4.71875), np.float32(0.0123), np.float32(3.1e-30), np.float32(1e30)):
        s = np.float32(a / np.float32(127.0))
        got = fp.div_f32(x, s)
        ref = x / s
        ok = np.isfinite(ref)
        assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


def test_sub_bf16_f32_matches_ieee_subtraction():
    rng = np.random.default_rng(9)
    k = W.f32_to_bf16_bits(_wide_f32(rng, 300_000, -135, 30))
    mu = _wide_f32(rng, 300_000, -140, 30)
    # include exact cancellations, zeros and wide exponent gaps
    mu[:1000] = W.bf16_bits_to_f32(k[:1000])
    mu[1000:2000] = 0.0
    k[2000:3000] = 0
    mu[3000:4000] = np.float32(3e-38)
    got = fp.sub_bf16_f32(k, mu)
    ref = W.bf16_bits_to_f32(k) - mu    # host binary32 subtraction
    assert np.array_equal(got, ref)
    # +0 for exact cancellation in round-to-nearest
    assert not np.signbit(got[:1000]).any()


def test_rne_to_int_matches_rint():
    rng = np.random.default_rng(3)
    q = (rng.uniform(-130, 130, 500_000)).astype(np.float32)
    q[:1000] = np.arange(-500, 500).astype(np.float32) + np.float32(0.5)   # exact ties
    q[1000:1100] = 0.0
    assert np.array_equal(fp.rne_to_int(q), np.rint(q).astype(np.int64))
    assert fp.rne_to_int(np.float32([2.5, -3.5, 0.5, -0.5, 1.5]).astype(np.float32)).tolist() == \
        [2, -4, 0, 0, 2]


# OCP 8-bit Floating Point Specification (OFP8), E4M3: bias 7, S.1111.111 is NaN,
# largest normal S.1111.110 = 448, smallest normal 2^-6, smallest subnormal 2^-9.
OCP_E4M3_TABLE = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
    0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x48: 4.0, 0x70: 128.0,
    0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0,
}


def test_e4m3_decode_ocp_table():
    for code, val in OCP_E4M3_TABLE.items():
        assert fp.e4m3_decode(np.uint8(code)) == val, hex(code)
    assert np.isnan(fp.e4m3_decode(np.uint8(0x7F))) and np.isnan(fp.e4m3_decode(np.uint8(0xFF)))


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(21)
    y = (rng.standard_normal(300_000) * np.exp2(rng.uniform(-14, 8.7, 300_000))).astype(np.float32)
    y = y[np.abs(y) < 464]
    # every rounding midpoint between consecutive finite codes, and the codes themselves
    pos = fp.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    extra = np.concatenate([mids, -mids, pos.astype(np.float32), np.float32([449.0, 463.9])])
    y = np.concatenate([y, extra.astype(np.float32)])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp.e4m3_encode(y)
    # torch keeps the sign of zero; so does the oracle
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    y = np.float32([448.0, 464.0, 500.0, 1e6, -1e6, -464.0])
    assert fp.e4m3_encode(y).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_bf16_parts_exact():
    bits = np.arange(65536, dtype=np.uint16)
    x = W.bf16_bits_to_f32(bits)
    fin = np.isfinite(x)
    neg, m, e = fp.bf16_parts(bits[fin])
    val = np.where(neg == 1, -1.0, 1.0) * np.ldexp(m.astype(np.float64), e.astype(np.int32))
    assert np.array_equal(val, x[fin].astype(np.float64))
    with pytest.raises(ValueError):
        fp.bf16_parts(np.uint16([0x7F80]))
