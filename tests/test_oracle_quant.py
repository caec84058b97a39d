"""Pins of the oracle's quantization steps (K mean, smoothing, INT8 and E4M3 codes).

Checked against exact rational arithmetic (Fraction brute force on tiny
inputs), closed forms and special cases (constant channels, symmetric data,
dyadic shifts, zero blocks, constructed ties), the host's IEEE binary32
arithmetic and torch's float8_e4m3fn conversion, and invariants of a
nearest-even quantizer (the absmax element maps to +-127, the reconstruction
error is at most half a scale step, codes stay in [-127, 127]).
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import fp, quant
import workloads as W


def _bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f(b):
    return W.bf16_bits_to_f32(b)


def _nearest(frac: Fraction, r):
    r = np.float32(r)
    dr = abs(Fraction(float(r)) - frac)
    for nb in (np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf))):
        dn = abs(Fraction(float(nb)) - frac)
        assert dr <= dn
        if dr == dn:
            assert int(r.view(np.uint32)) & 1 == 0


# --------------------------------------------------------------------------- K mean

def test_kmean_is_nearest_binary32_of_exact_mean():
    rng = np.random.default_rng(0)
    for N in (1, 2, 3, 7, 64, 129):
        x = rng.standard_normal((N, 5)) * np.exp2(rng.uniform(-30, 30, (N, 5)))
        k = _bf16(x)
        mu = quant.kmean_exact(k)
        for c in range(5):
            exact = sum(Fraction(float(v)) for v in _f(k[:, c])) / N
            _nearest(exact, mu[c])


def test_kmean_closed_forms():
    # a constant channel has that constant as its mean, exactly
    k = _bf16(np.tile(np.float32([1.5, -3.25, 0.0, 2.0 ** -100]), (1000, 1)))
    assert np.array_equal(quant.kmean_exact(k), np.float32([1.5, -3.25, 0.0, 2.0 ** -100]))
    # symmetric data has mean 0
    rng = np.random.default_rng(1)
    half = _bf16(rng.standard_normal((500, 8)))
    sym = np.concatenate([half, half ^ np.uint16(0x8000)])
    assert np.all(quant.kmean_exact(sym) == 0)
    # adding a dyadic constant that keeps every value exact shifts the mean by it
    base = _bf16(rng.integers(-64, 64, (300, 4)).astype(np.float32) / 8)
    shifted = _bf16(_f(base) + np.float32(4.0))
    assert np.array_equal(_f(shifted) - _f(base), np.full((300, 4), 4.0, np.float32))
    assert np.array_equal(quant.kmean_exact(shifted), quant.kmean_exact(base) + np.float32(4.0))
    # the sum of N copies of 1/3-ish values: mean of {a, b} = (a+b)/2 exactly when representable
    two = _bf16(np.float32([[1.0], [2.0]]))
    assert quant.kmean_exact(two)[0] == np.float32(1.5)
    # order independence (a float reduction would not be)
    perm = rng.permutation(300)
    assert np.array_equal(quant.kmean_exact(base[perm]), quant.kmean_exact(base))


def test_kmean_cancellation_is_exact():
    # huge values that cancel plus one small value: any float accumulation loses the small one
    k = _bf16(np.float32([[2.0 ** 60], [1.0], [-(2.0 ** 60)]]))
    assert quant.kmean_exact(k)[0] == np.float32(1.0 / 3.0)


# --------------------------------------------------------------------------- smoothing

def test_smooth_k_matches_ieee():
    rng = np.random.default_rng(2)
    k = _bf16(rng.standard_normal((2000, 64)) + rng.normal(0, 2 ** 0.5, 64))
    mu = quant.kmean_exact(k)
    assert np.array_equal(quant.smooth_k(k, mu), _f(k) - mu[None, :])


# --------------------------------------------------------------------------- INT8 codes

def test_block_absmax_and_scale_definition():
    rng = np.random.default_rng(3)
    x = _f(_bf16(rng.standard_normal((300, 16))))
    a = quant.block_absmax(x, 64)
    assert a.shape == (5,)
    for i in range(5):
        assert a[i] == np.abs(x[i * 64:(i + 1) * 64]).max()
    s = quant.scales_from_absmax(a, 127.0)
    for ai, si in zip(a, s):
        _nearest(Fraction(float(ai)) / 127, si)
    assert quant.scales_from_absmax(np.float32([0.0]), 127.0)[0] == 0.0


def test_codes_match_ieee_rint_of_quotient():
    rng = np.random.default_rng(4)
    x = _f(_bf16(rng.standard_normal((1024, 128)) * 3))
    s = quant.scales_from_absmax(quant.block_absmax(x, 128), 127.0)
    srow = np.repeat(s, 128)
    got = quant.codes_i8(x, srow)
    ref = np.clip(np.rint(x / srow[:, None]), -127, 127).astype(np.int8)   # host IEEE division
    assert np.array_equal(got, ref)


def test_codes_exhaustive_bf16_inputs():
    bits = np.arange(65536, dtype=np.uint16)
    x = _f(bits)
    x = x[np.isfinite(x)].reshape(-1, 1)
    for a in (np.float32(4.84375), np.float32(0.75), np.float32(200.0)):
        s = np.float32(a / np.float32(127.0))
        with np.errstate(over="ignore"):
            ref = np.clip(np.rint(x / s), -127, 127).astype(np.int8)
        got = quant.codes_i8(x, np.full(x.shape[0], s, np.float32))
        assert np.array_equal(got, ref)


def test_codes_constructed_ties_and_zero_block():
    s = np.float32(1.0)
    x = np.float32([[2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.5, 1000.0]])
    assert quant.codes_i8(x, np.float32([s])).tolist() == [[2, -4, 0, 0, 2, 126, -127, 127]]
    z = np.zeros((64, 8), np.float32)
    qc, qs = quant.quantize_q(_bf16(z), 64)
    assert qs.tolist() == [0.0] and not qc.any()


def test_quantizer_invariants():
    rng = np.random.default_rng(5)
    for dist in ("normal", "t3"):
        raw = rng.standard_normal((777, 128)) if dist == "normal" else rng.standard_t(3, (777, 128))
        qb = _bf16(raw)
        qc, qs = quant.quantize_q(qb, 128)
        x = _f(qb)
        assert qc.min() >= -127 and qc.max() <= 127
        for i in range(qs.size):
            blk = x[i * 128:(i + 1) * 128]
            cb = qc[i * 128:(i + 1) * 128].astype(np.float64)
            j = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert abs(cb[j]) == 127 and np.sign(cb[j]) == np.sign(blk[j])
            err = np.abs(blk.astype(np.float64) - cb * float(qs[i]))
            # |x/s| <= 127 (plus rounding of s); the binary32 quotient is off by at most
            # 2^-24 relative, then rne moves it by at most 1/2
            assert err.max() <= float(qs[i]) * (0.5 + 128 * 2.0 ** -24)


def test_quantize_k_uses_smoothed_values():
    rng = np.random.default_rng(6)
    kb = _bf16(rng.standard_normal((200, 32)) + 5.0)      # large common offset
    kc, ks, mu = quant.quantize_k(kb, 64)
    assert np.all(np.abs(mu - 5.0) < 0.5)
    x = _f(kb) - mu[None, :]
    ref_s = quant.scales_from_absmax(quant.block_absmax(x, 64), 127.0)
    assert np.array_equal(ks, ref_s)
    srow = np.repeat(ks, 64)[:200]
    assert np.array_equal(kc, np.clip(np.rint(x / srow[:, None]), -127, 127).astype(np.int8))


def test_block_permutation_permutes_codes():
    rng = np.random.default_rng(7)
    kb = _bf16(rng.standard_normal((256, 64)) + 1.0)
    kc, ks, mu = quant.quantize_k(kb, 64)
    order = np.array([2, 0, 3, 1])
    perm = np.concatenate([np.arange(64) + 64 * o for o in order])
    kc2, ks2, mu2 = quant.quantize_k(kb[perm], 64)
    assert np.array_equal(mu2, mu) and np.array_equal(ks2, ks[order])
    assert np.array_equal(kc2, kc[perm])


# --------------------------------------------------------------------------- FP8 V

def _check_pow2_scale(a, s, emin=-127):
    """s = 2^e is the smallest power of two (>= 2^emin) with a <= 448 s,
    checked in exact rationals."""
    m, e = np.frexp(np.float64(s))
    assert m == 0.5, s                                        # a power of two
    e = int(e) - 1
    a = Fraction(float(a))
    assert a <= 448 * Fraction(2) ** e
    assert e == emin or a > 448 * Fraction(2) ** (e - 1)


def test_v_fp8_matches_ieee_and_torch():
    rng = np.random.default_rng(8)
    # blocks of very different magnitude, including ones whose absmax sits
    # on, just above and just below 448 times a power of two
    x = rng.standard_normal((320, 64)) * np.exp2(rng.integers(-30, 30, size=5)).repeat(64)[:, None]
    x[70, 3] = 448.0 * 2.0 ** 5
    x[140, 9] = 448.0 * 2.0 ** -3 * (1 + 2.0 ** -7)
    x[200, 1] = -448.0 * (1 - 2.0 ** -8)
    vb = _bf16(x)
    vc, vs = quant.quantize_v_fp8(vb, 64)
    x = _f(vb)
    for i in range(vs.size):
        _check_pow2_scale(np.abs(x[i * 64:(i + 1) * 64]).max(), vs[i])
    srow = np.repeat(vs, 64)[:320][:, None]
    y = x / srow                                              # host IEEE division (exact: a power of two)
    ref = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(vc, ref)
    # the absmax element of each block lands in the top binade of E4M3:
    # (224, 448], codes 0x77 .. 0x7E by magnitude (0x76 = 224 itself when it
    # rounds down)
    for i in range(vs.size):
        blk = np.abs(x[i * 64:(i + 1) * 64])
        j = np.unravel_index(blk.argmax(), blk.shape)
        assert 0x76 <= (vc[i * 64 + j[0], j[1]] & 0x7F) <= 0x7E
    # reconstruction within half an E4M3 step (relative 2^-4) or half the subnormal step
    deq = fp.e4m3_decode(vc) * srow
    tol = np.maximum(np.abs(x) * 2.0 ** -4, srow * 2.0 ** -10)
    assert np.all(np.abs(deq - x) <= tol * (1 + 1e-6))


def test_v_fp8_scale_edges():
    # absmax exactly 448 * 2^e gives 2^e (code 448), one bf16 step above gives
    # 2^(e+1); blocks too small for 2^-127 clamp there
    for e in (-20, 0, 7):
        for bump, want in ((0, e), (1, e + 1)):
            a = np.float32(448.0 * 2.0 ** e)
            bits = (np.array([a], np.float32).view(np.uint32) >> 16).astype(np.uint16) + bump
            vb = np.zeros((64, 8), np.uint16)
            vb[5, 2] = bits[0]
            vc, vs = quant.quantize_v_fp8(vb, 64)
            assert vs[0] == np.float32(2.0 ** want), (e, bump, vs)
            assert vc[5, 2] == (0x7E if bump == 0 else 0x76)   # 448, or 448.x / 2 rounded to 224
    tiny = np.zeros((64, 8), np.uint16)
    tiny[0, 0] = 0x0001                                         # smallest bf16 subnormal, 2^-133
    vc, vs = quant.quantize_v_fp8(tiny, 64)
    assert vs[0] == np.float32(2.0 ** -127)
    _check_pow2_scale(2.0 ** -133, vs[0])


def test_v_fp8_zero_block():
    vb = np.zeros((64, 8), np.uint16)
    vc, vs = quant.quantize_v_fp8(vb, 64)
    assert vs.tolist() == [0.0] and not vc.any()
