"""Pins of the oracle's W8A8 block-wise INT8 linear layer (oracle/w8a8.py).

What ties it to something other than itself:
  * planted inputs: x and W built as code * 2^e with a distinct power-of-two
    scale per 128x128 block and a +-127 code in every block are exactly what
    the quantizer must return (codes and scales), and for them the layer must
    equal the exact product x W^T + b computed in integers;
  * nearest-even ties and the +-127 clamp on constructed values;
  * each scale is the binary32 number nearest to absmax/127 (Fraction brute force);
  * the 8-bit rounding error bound against the unquantized product on random
    data (a dropped term, a wrong scale index or a transposed operand breaks it);
  * permutations of rows inside a block and of the K slices, zero blocks, bias.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import w8a8
import workloads as W
from workloads import linear as WL


def _planted(R, C, rng, exps, zero_block=None):
    """codes int [R, C] with a +-127 in every 128x128 block, scales 2^e per
    block (exps [rb, cb]), x = codes * scale as float32 (exact in bf16)."""
    rb, cb = -(-R // 128), C // 128
    codes = rng.integers(-127, 128, size=(R, C))
    scales = np.ldexp(1.0, exps).astype(np.float32)
    for i in range(rb):
        for j in range(cb):
            r0, r1 = 128 * i, min(R, 128 * (i + 1))
            if zero_block == (i, j):
                codes[r0:r1, 128 * j:128 * (j + 1)] = 0
                scales[i, j] = 0.0
                continue
            rr = rng.integers(r0, r1)
            cc = rng.integers(128 * j, 128 * (j + 1))
            codes[rr, cc] = 127 if rng.integers(2) else -127
    srow = np.repeat(scales, 128, axis=0)[:R]
    s = np.repeat(srow, 128, axis=1)
    x = (codes * s.astype(np.float64)).astype(np.float32)
    # bf16 round trip is the identity on these values
    assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)), x)
    return codes.astype(np.int8), scales, x


def test_quantizer_returns_planted_codes_and_scales():
    rng = np.random.default_rng(10)
    R, C = 300, 384
    exps = rng.integers(-6, 5, size=(3, 3))
    codes, scales, x = _planted(R, C, rng, exps, zero_block=(1, 2))
    c, s = w8a8.quantize_blocks(x)
    assert s.shape == (3, 3) and c.shape == (R, C)
    np.testing.assert_array_equal(s, scales)
    np.testing.assert_array_equal(c, codes)


def test_layer_is_exact_product_on_representable_inputs():
    rng = np.random.default_rng(11)
    M, K, N = 300, 384, 200
    cx, sx, x = _planted(M, K, rng, rng.integers(-4, 4, size=(3, 3)))
    cw, sw, wt = _planted(N, K, rng, rng.integers(-4, 4, size=(2, 3)))
    b = (rng.integers(-64, 64, size=N) / 8.0).astype(np.float32)
    qx, qsx = w8a8.quantize_blocks(x)
    qw, qsw = w8a8.quantize_blocks(wt)
    y = w8a8.linear(qx, qsx, qw, qsw, b)
    # exact: x * 2^4 and W * 2^4 are integers (exponents >= -4)
    xi = (x.astype(np.float64) * 16).astype(np.int64)
    wi = (wt.astype(np.float64) * 16).astype(np.int64)
    assert np.array_equal(xi / 16.0, x) and np.array_equal(wi / 16.0, wt)
    exact = [[Fraction(int(v), 256) for v in row] for row in (xi @ wi.T)]
    for m in range(0, M, 7):
        for n in range(0, N, 5):
            assert Fraction(float(y[m, n])) == exact[m][n] + Fraction(float(b[n]))


def test_nearest_even_ties_and_clamp():
    # block absmax 127 * 2^-2 -> s = 2^-2 exactly; values at k + 1/2 steps tie
    x = np.zeros((128, 128), np.float32)
    x[0, 0] = 127 * 0.25
    vals = {1: 2.5, 2: 3.5, 3: -2.5, 4: 0.5, 5: 1.5, 6: -0.5, 7: 126.5}
    for c, v in vals.items():
        x[0, c] = v * 0.25
    c, s = w8a8.quantize_blocks(x)
    assert s[0, 0] == np.float32(0.25)
    want = {1: 2, 2: 4, 3: -2, 4: 0, 5: 2, 6: 0, 7: 126}
    for col, code in want.items():
        assert c[0, col] == code
    assert c[0, 0] == 127


def test_scales_are_nearest_binary32_of_absmax_over_127():
    rng = np.random.default_rng(12)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((200, 256)).astype(np.float32) * 3))
    c, s = w8a8.quantize_blocks(x)
    for i in range(2):
        for j in range(2):
            blk = x[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            a = Fraction(float(np.abs(blk).max())) / 127
            r = s[i, j]
            lo = np.nextafter(r, np.float32(0))
            hi = np.nextafter(r, np.float32(np.inf))
            d = abs(Fraction(float(r)) - a)
            assert d <= abs(Fraction(float(lo)) - a) and d <= abs(Fraction(float(hi)) - a)
            # the block's absmax element maps to +-127
            k = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert abs(int(c[128 * i + k[0], 128 * j + k[1]])) == 127


def test_error_bound_against_unquantized_product():
    rng = np.random.default_rng(13)
    M, K, N = 260, 512, 140
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    wt = W.bf16_bits_to_f32(W.f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)))
    cx, sx = w8a8.quantize_blocks(x)
    cw, sw = w8a8.quantize_blocks(wt)
    y = w8a8.linear(cx, sx, cw, sw)
    ref = x.astype(np.float64) @ wt.astype(np.float64).T
    # code = rne(fl32(v / s)): the quotient's own rounding (half an ulp of a
    # value below 128, at most 2^-17) adds to the half step, so
    # |v - s c| <= s (1/2 + 2^-17) per element
    h = 0.5 + 2.0 ** -17
    SX = np.repeat(np.repeat(sx.astype(np.float64), 128, 0)[:M], 128, 1) * h
    SW = np.repeat(np.repeat(sw.astype(np.float64), 128, 0)[:N], 128, 1) * h
    assert np.all(np.abs(x - SX / h * cx) <= SX)
    assert np.all(np.abs(wt - SW / h * cw) <= SW)
    bound = np.abs(x) @ SW.T + SX @ np.abs(wt).T + SX @ SW.T
    err = np.abs(y - ref)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    # and the bound is not vacuous: the error is small against the output scale
    assert err.max() < 0.05 * np.abs(ref).max()


def test_row_and_slice_permutations():
    rng = np.random.default_rng(14)
    M, K, N = 256, 384, 96
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    wt = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32)))
    cw, sw = w8a8.quantize_blocks(wt)
    cx, sx = w8a8.quantize_blocks(x)
    y = w8a8.linear(cx, sx, cw, sw)
    # rows permuted inside each 128-row block: same codes permuted, rows of y permuted
    p = np.concatenate([rng.permutation(128), 128 + rng.permutation(128)])
    cxp, sxp = w8a8.quantize_blocks(x[p])
    np.testing.assert_array_equal(sxp, sx)
    np.testing.assert_array_equal(w8a8.linear(cxp, sxp, cw, sw), y[p])
    # the same permutation of the 128-wide K slices on both sides leaves y unchanged
    q = np.concatenate([np.arange(128) + 128 * j for j in (2, 0, 1)])
    cxq, sxq = w8a8.quantize_blocks(x[:, q])
    cwq, swq = w8a8.quantize_blocks(wt[:, q])
    np.testing.assert_allclose(w8a8.linear(cxq, sxq, cwq, swq), y, rtol=1e-13, atol=1e-12)


def test_zero_block_and_bias():
    rng = np.random.default_rng(15)
    M, K, N = 128, 256, 64
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, 128:] = 0
    wt = rng.standard_normal((N, K)).astype(np.float32)
    cx, sx = w8a8.quantize_blocks(x)
    assert sx[0, 1] == 0 and not cx[:, 128:].any()
    cw, sw = w8a8.quantize_blocks(wt)
    b = rng.standard_normal(N).astype(np.float32)
    y0 = w8a8.linear(cx, sx, cw, sw)
    yb = w8a8.linear(cx, sx, cw, sw, b)
    np.testing.assert_allclose(yb - y0, np.broadcast_to(b.astype(np.float64), yb.shape), rtol=0, atol=1e-12)
    # only the first K slice contributes
    c1, s1 = w8a8.quantize_blocks(x[:, :128])
    cw1, sw1 = w8a8.quantize_blocks(wt[:, :128])
    np.testing.assert_array_equal(w8a8.linear(c1, s1, cw1, sw1), y0)
    # the bound is the sum of the absolute terms
    bd = w8a8.linear_bound(cx, sx, cw, sw, b)
    assert np.all(bd >= np.abs(yb) - 1e-9)


def test_columns_must_fill_blocks():
    with pytest.raises(ValueError):
        w8a8.quantize_blocks(np.zeros((4, 100), np.float32))


def test_workload_generator_block_streams():
    w = WL.get_linear("w8a8-tiny")
    x = WL.gen_x(w)
    assert x.shape == (w.M, w.K) and x.dtype == np.uint16
    np.testing.assert_array_equal(WL.gen_x_blocks(w, [2, 0]), np.concatenate([x[256:], x[:128]]))
    wt = WL.gen_w(w)
    assert wt.shape == (w.N, w.K)
    v = W.bf16_bits_to_f32(wt).astype(np.float64)
    assert abs(v.std() * np.sqrt(w.K) - 1) < 0.05
    blocks = WL.checked_row_blocks(WL.get_linear("w8a8-qkv-wan14b-480p"))
    assert blocks[-1] == -(-32760 // 128) - 1 and len(set(blocks)) == 4
