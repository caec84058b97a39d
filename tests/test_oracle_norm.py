"""Pins of the oracle's RMSNorm + INT8 block quantization (oracle/norm.py).

  * mu2 is the binary32 number nearest to the exact mean square (Fraction
    brute force, subnormal and large inputs included);
  * y is within a few binary32 roundings of the float64 RMSNorm;
  * power-of-two scaling of a row leaves y and the codes unchanged and scales
    r by the inverse power (exact when eps is negligible);
  * a constant row normalizes to +-gamma; permuting the columns (with gamma)
    permutes y exactly (the exact sum does not depend on the order).
"""
from fractions import Fraction

import numpy as np

from oracle import fp, norm, w8a8
import workloads as W


def _bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def _f(b):
    return W.bf16_bits_to_f32(b)


def _is_nearest_f32(r, exact: Fraction):
    r = np.float32(r)
    d = abs(Fraction(float(r)) - exact)
    for nb in (np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf))):
        dn = abs(Fraction(float(nb)) - exact)
        assert d <= dn
        if d == dn:
            assert int(r.view(np.uint32)) & 1 == 0


def test_mean_square_is_nearest_binary32():
    rng = np.random.default_rng(0)
    rows = [rng.standard_normal(256) * 3,
            np.concatenate([rng.standard_normal(200) * 1e-39, rng.standard_normal(56)]),   # subnormals
            rng.standard_normal(256) * 1e15,
            np.concatenate([[6e4], rng.standard_normal(255) * 1e-30]),
            np.full(256, 0.0)]
    x = np.stack([_bits(r) for r in rows])
    mu2, r = norm.rms_inverse(x, 1e-6)
    for i in range(len(rows)):
        exact = sum(Fraction(float(v)) ** 2 for v in _f(x[i])) / 256
        _is_nearest_f32(mu2[i], exact)
    assert mu2[4] == 0 and r[4] == np.float32(1) / np.sqrt(np.float32(1e-6))


def test_close_to_float64_rmsnorm():
    rng = np.random.default_rng(1)
    x = _bits(rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1)))
    g = (rng.standard_normal(512) * 0.5 + 1).astype(np.float32)
    y, r = norm.rmsnorm(x, g, 1e-6)
    xf = _f(x).astype(np.float64)
    ref = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + np.float64(np.float32(1e-6))) * g.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 6 * 2.0 ** -24 * np.abs(ref) + 1e-30)


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((130, 384)).astype(np.float32)
    g = (rng.standard_normal(384) + 1).astype(np.float32)
    eps = 2.0 ** -140   # far below every mean square here
    c0, s0, r0 = norm.rmsnorm_quantize(_bits(x), g, eps)
    c1, s1, r1 = norm.rmsnorm_quantize(_bits(x * 256), g, eps)
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s0, s1)
    np.testing.assert_array_equal(r1 * np.float32(256), r0)


def test_constant_rows_and_column_permutation():
    rng = np.random.default_rng(3)
    g = (rng.standard_normal(256) + 1).astype(np.float32)
    x = np.zeros((3, 256), np.float32)
    x[0] = 0.75
    x[1] = -3.0
    x[2] = rng.standard_normal(256)
    y, r = norm.rmsnorm(_bits(x), g, 2.0 ** -140)
    np.testing.assert_array_equal(y[0], g)   # fl32(0.75 * fl32(1/0.75)) is exactly 1
    np.testing.assert_array_equal(y[1], -g)
    p = rng.permutation(256)
    yp, _ = norm.rmsnorm(_bits(x[:, p]), g[p], 2.0 ** -140)
    np.testing.assert_array_equal(yp, y[:, p])


def test_quantize_matches_block_rule():
    rng = np.random.default_rng(4)
    x = _bits(rng.standard_normal((200, 256)))
    c, s, r = norm.rmsnorm_quantize(x, None, 1e-6)
    y, r2 = norm.rmsnorm(x, None, 1e-6)
    c2, s2 = w8a8.quantize_blocks(y)
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(r, r2)


def test_mean_square_next_to_a_midpoint():
    """Crafted rows (tests/norm_cases.py) whose exact mean square is, by
    construction, exactly on, just above or just below the midpoint of two
    adjacent binary32 numbers, the deciding squares lying 2^150 and 2^300
    below the row's largest: the oracle's mean square must be the intended
    neighbour (even one for the tie) and the nearest binary32 by brute force."""
    import norm_cases as NC
    for i, kind in enumerate(NC.KINDS):
        bits, lo, hi, want = NC.mean_square_row(kind, seed=11 * i)
        exact = NC.exact_mean_square(bits)
        mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
        side = {"even": 0, "hi": 1, "lo": -1}[NC.KINDS[kind]]
        assert (exact > mid) - (exact < mid) == side, kind
        mu2, r = norm.rms_inverse(bits[None, :], NC.EPS)
        assert mu2[0] == want, kind
        _is_nearest_f32(mu2[0], exact)
        for reps in (2, 4):      # tiled rows: same mean square
            mu2t, _ = norm.rms_inverse(np.tile(bits, reps)[None, :], NC.EPS)
            assert mu2t[0] == want, kind


def test_f32_to_bf16_matches_torch_rounding():
    """The oracle's integer-decided nearest-even rounding to bf16 against
    torch's CPU float32 -> bfloat16 conversion (an independent routine), on
    random values over the whole binary32 range, exact ties in both
    directions, values next to the overflow threshold, subnormals, zeros and
    infinities; NaN stays a NaN of the same sign."""
    import torch
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 2000, dtype=np.uint32) << 16) | 0x8000
    edge = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0x00000001, 0x80000000, 0,
                     0x7F800000, 0xFF800000, 0x7FC00000, 0x3F808000, 0x3F818000], np.uint32)
    bits = np.concatenate([u, ties, edge])
    bits = bits[(bits & 0x7FFFFFFF) <= 0x7F800000]             # finite or infinite
    y = bits.view(np.float32)
    got = fp.f32_to_bf16(y)
    ref = torch.from_numpy(y.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    # NaN (torch writes its own pattern): a NaN of the same sign
    nan = np.array([0x7FC00000, 0xFFC00001, 0x7F800001], np.uint32)
    nb = fp.f32_to_bf16(nan.view(np.float32)).astype(np.uint32)
    assert np.all((nb & 0x7F80) == 0x7F80) and np.all((nb & 0x7F) != 0)
    np.testing.assert_array_equal(nb >> 15, nan >> 31)


def test_qk_rmsnorm_rows_are_tokens():
    """qk_rmsnorm normalizes each token over its H*d values: the same as
    rmsnorm on the [B*N, H*d] token rows, rounded to bf16; and scaling one
    token by a power of two leaves every output unchanged."""
    rng = np.random.default_rng(6)
    B, H, N, d = 2, 3, 5, 64
    x = _bits(rng.standard_normal((B, H, N, d)) * rng.uniform(0.1, 10, (B, 1, N, 1)))
    g = (rng.standard_normal(H * d) * 0.2 + 1).astype(np.float32)
    out = norm.qk_rmsnorm(x, g, 1e-6)
    rows = x.transpose(0, 2, 1, 3).reshape(B * N, H * d)
    y, _ = norm.rmsnorm(rows, g, 1e-6)
    want = fp.f32_to_bf16(y).reshape(B, N, H, d).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(out, want)
    x2 = x.copy()
    x2[1, :, 3, :] = _bits(_f(x[1, :, 3, :]) * np.float32(2.0 ** 10))
    np.testing.assert_array_equal(norm.qk_rmsnorm(x2, g, 2.0 ** -140), norm.qk_rmsnorm(x, g, 2.0 ** -140))


# ---------------------------------------------------------------------------
# LayerNorm
# ---------------------------------------------------------------------------

def _ln_rows():
    rng = np.random.default_rng(7)
    rows = [rng.standard_normal(256) * 3 + 5,
            rng.standard_normal(256) * 1e-3 - 40.0,                        # mean far above the spread
            np.concatenate([[1e18, -3e17], rng.standard_normal(254) * 1e-30]),
            np.concatenate([rng.standard_normal(200) * 1e-39, rng.standard_normal(56) * 1e-36]),  # subnormals
            np.full(256, -2.5),
            rng.standard_normal(256) * 1e15]
    return np.stack([_bits(r) for r in rows])


def test_layernorm_stats_are_nearest_binary32():
    x = _ln_rows()
    mu, var, r = norm.layernorm_stats(x, 1e-6)
    K = x.shape[1]
    for i in range(x.shape[0]):
        vals = [Fraction(float(v)) for v in _f(x[i])]
        _is_nearest_f32(mu[i], sum(vals) / K)
        d = (_f(x[i]) - mu[i]).astype(np.float32)                  # binary32 differences
        _is_nearest_f32(var[i], sum(Fraction(float(v)) ** 2 for v in d) / K)
    assert var[4] == 0 and mu[4] == np.float32(-2.5)


def test_layernorm_close_to_float64():
    rng = np.random.default_rng(8)
    x = _bits(rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1)) + rng.uniform(-1, 1, (64, 1)))
    g = (rng.standard_normal(512) * 0.5 + 1).astype(np.float32)
    b = (rng.standard_normal(512) * 0.1).astype(np.float32)
    y, _, _ = norm.layernorm(x, g, b, 1e-6)
    xf = _f(x).astype(np.float64)
    m = xf.mean(axis=1, keepdims=True)
    ref = (xf - m) / np.sqrt(((xf - m) ** 2).mean(axis=1, keepdims=True) + np.float64(np.float32(1e-6)))
    ref = ref * g.astype(np.float64) + b.astype(np.float64)
    scale = np.abs(xf - m).max(axis=1, keepdims=True) / np.sqrt(((xf - m) ** 2).mean(axis=1, keepdims=True))
    assert np.all(np.abs(y - ref) <= 2.0 ** -20 * (scale * np.abs(g) + np.abs(b)) + 1e-30)


def test_layernorm_power_of_two_scaling_and_constant_rows():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((130, 384)).astype(np.float32) + 0.5
    g = (rng.standard_normal(384) + 1).astype(np.float32)
    b = (rng.standard_normal(384) * 0.2).astype(np.float32)
    eps = 2.0 ** -140
    c0, s0, m0, r0 = norm.layernorm_quantize(_bits(x), g, b, eps)
    c1, s1, m1, r1 = norm.layernorm_quantize(_bits(x * 1024), g, b, eps)
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s0, s1)
    np.testing.assert_array_equal(m1, m0 * np.float32(1024))
    np.testing.assert_array_equal(r1 * np.float32(1024), r0)
    y, _, _ = norm.layernorm(_bits(np.full((2, 256), 3.0, np.float32)), g[:256], b[:256], 1e-6)
    np.testing.assert_array_equal(y, np.broadcast_to(b[:256], (2, 256)))     # d = 0: y = beta
    c, s, _, _ = norm.layernorm_quantize(_bits(x), g, b, 1e-6)
    y2, _, _ = norm.layernorm(_bits(x), g, b, 1e-6)
    c2, s2 = w8a8.quantize_blocks(y2)
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(s, s2)


def test_layernorm_variance_next_to_a_midpoint():
    """Rows [x, -x] with x a crafted RMS row (tests/norm_cases.py): the exact
    mean is 0, so d = x and the variance is the crafted mean square, which
    lies exactly on, just above or just below a binary32 midpoint with the
    deciding squares 2^150 and 2^300 below the largest."""
    import norm_cases as NC
    for i, kind in enumerate(NC.KINDS):
        bits, lo, hi, want = NC.mean_square_row(kind, seed=11 * i)
        row = np.concatenate([bits, bits ^ np.uint16(0x8000)])
        mu, var, _ = norm.layernorm_stats(row[None, :], NC.EPS)
        assert mu[0] == 0 and var[0] == want, kind
