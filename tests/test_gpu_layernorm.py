"""GPU parity of LayerNorm fused with the W8A8 block quantization
(sqattn_w8a8_layernorm_quantize / sqattn_w8a8_linear_layernorm) against
oracle/norm.py: mean, inverse standard deviation, codes and scales bit for
bit; the fused linear equals quantize + gemm bit for bit."""
import math

import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import dev_bf16, host
from oracle import norm
from workloads import linear as WL

pytestmark = pytest.mark.gpu


def _rows(R, C, seed, kind):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, C)) * rng.uniform(0.05, 20, (R, 1)) + rng.uniform(-3, 3, (R, 1))
    if kind == "spread":
        x = x * np.ldexp(1.0, rng.integers(-60, 61, R))[:, None]
        x[0] = 0.0                                                   # zero row: rstd = 1/sqrt(eps)
        if R > 5:
            x[1, : C // 2] = rng.standard_normal(C // 2) * 1e-39      # subnormals beside normal values
            x[2] = rng.standard_normal(C) * 1e37 * 3                  # variance overflows: rstd = 0
            x[3] = rng.standard_normal(C) * 1e-3 + 1e4                # mean far above the spread
            x[4] = -7.25                                              # constant row: d = 0
            x[5, ::2] = -x[5, 1::2]                                   # a row summing to zero
        x[-1, ::7] = 0.0
    return W.f32_to_bf16_bits(x.astype(np.float32))


def _check(xb, gamma, beta, eps, codes, scales, mu, r):
    c_ref, s_ref, m_ref, r_ref = norm.layernorm_quantize(xb, gamma, beta, eps)
    assert np.array_equal(host(mu).view(np.uint32), m_ref.view(np.uint32)), "mean differs"
    assert np.array_equal(host(r).view(np.uint32), r_ref.view(np.uint32)), "rstd differs"
    assert np.array_equal(host(scales).view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    assert np.array_equal(host(codes), c_ref), "codes differ"


def _dev(a):
    return None if a is None else torch.from_numpy(a).cuda()


@pytest.mark.parametrize("R,C", [(300, 384), (1, 128), (129, 640), (1000, 5120)])
@pytest.mark.parametrize("kind", ["normal", "spread"])
@pytest.mark.parametrize("affine", ["none", "gamma", "both"])
def test_layernorm_quantize_bit_exact(R, C, kind, affine):
    print(f"case layernorm R={R} C={C} kind={kind} affine={affine}", flush=True)
    xb = _rows(R, C, seed=R + C + len(affine), kind=kind)
    rng = np.random.default_rng(C)
    g = (rng.standard_normal(C) * 0.3 + 1).astype(np.float32) if affine != "none" else None
    b = (rng.standard_normal(C) * 0.2).astype(np.float32) if affine == "both" else None
    eps = 1e-6
    codes, scales, mu, r = sq.w8a8_layernorm_quantize(dev_bf16(xb), _dev(g), _dev(b), eps)
    torch.cuda.synchronize()
    _check(xb, g, b, eps, codes, scales, mu, r)


def test_variance_next_to_a_midpoint():
    """Rows [x, -x] with x a crafted RMS row (tests/norm_cases.py): the mean is
    exactly 0 and the variance is the crafted mean square, on, just above or
    just below a binary32 midpoint with the deciding squares two levels
    down; also tiled 4 times (same variance, every level sum scaled by 4)."""
    import norm_cases as NC
    rows = [NC.mean_square_row(kind, seed=11 * i) for i, kind in enumerate(NC.KINDS)]
    x1 = np.stack([np.concatenate([b, b ^ np.uint16(0x8000)]) for b, _, _, _ in rows])
    want = np.array([w for _, _, _, w in rows], np.float32)
    for xb in (x1, np.tile(x1, (1, 4))):
        print(f"case layernorm midpoint rows R={xb.shape[0]} C={xb.shape[1]}", flush=True)
        codes, scales, mu, r = sq.w8a8_layernorm_quantize(dev_bf16(xb), None, None, NC.EPS)
        torch.cuda.synchronize()
        _check(xb, None, None, NC.EPS, codes, scales, mu, r)
        assert not host(mu).any()
        assert np.array_equal(host(r), np.float32(1) / np.sqrt(want + np.float32(NC.EPS)))


def test_linear_layernorm_equals_quantize_then_gemm():
    M, N, K = 700, 640, 2560
    rng = np.random.default_rng(3)
    X = dev_bf16(_rows(M, K, seed=4, kind="normal"))
    wb = W.f32_to_bf16_bits((rng.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32))
    wc, ws = sq.w8a8_quantize(dev_bf16(wb))
    g = torch.from_numpy((rng.standard_normal(K) * 0.2 + 1).astype(np.float32)).cuda()
    be = torch.from_numpy((rng.standard_normal(K) * 0.1).astype(np.float32)).cuda()
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).cuda()
    y1 = sq.w8a8_linear_layernorm(X, wc, ws, gamma=g, beta=be, eps=1e-6, bias=b, out_dtype=torch.bfloat16)
    xc, xs, _, _ = sq.w8a8_layernorm_quantize(X, g, be, 1e-6)
    y2 = sq.w8a8_gemm(xc, xs, wc, ws, bias=b, out_dtype=torch.bfloat16)
    y3 = sq.w8a8_linear_layernorm(X, wc, ws, gamma=g, beta=be, eps=1e-6, bias=b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_full_size_qkv_input():
    """The 14B QKV projection input (32760 x 5120) with a DiT modulation
    (gamma = 1 + scale, beta = shift): codes and scales of the sampled row
    blocks, mean and rstd of their rows."""
    w = WL.get_linear("w8a8-qkv-wan14b-480p")
    print(f"case layernorm full M={w.M} K={w.K}", flush=True)
    x = WL.gen_x(w)
    rng = np.random.default_rng(6)
    g = (1 + rng.standard_normal(w.K) * 0.2).astype(np.float32)
    b = (rng.standard_normal(w.K) * 0.1).astype(np.float32)
    codes, scales, mu, r = sq.w8a8_layernorm_quantize(dev_bf16(x), _dev(g), _dev(b), 1e-6)
    torch.cuda.synchronize()
    blocks = WL.checked_row_blocks(w)
    rows = np.concatenate([np.arange(128 * i, min(w.M, 128 * i + 128)) for i in blocks])
    c_ref, s_ref, m_ref, r_ref = norm.layernorm_quantize(x[rows], g, b, 1e-6)
    assert np.array_equal(host(mu)[rows].view(np.uint32), m_ref.view(np.uint32))
    assert np.array_equal(host(r)[rows].view(np.uint32), r_ref.view(np.uint32))
    assert np.array_equal(host(scales)[blocks].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(codes)[rows], c_ref)


def test_empty_rows():
    X = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    codes, scales, mu, r = sq.w8a8_layernorm_quantize(X)
    torch.cuda.synchronize()
    assert codes.shape == (0, 256) and mu.shape == (0,)


def test_long_rows_fill_the_windows():
    """Rows of 131072 values of the largest significand: the mean's 64-bit
    window and the squares' 128-bit window fill at their top and must be
    emptied before they overflow; one row adds a large offset (its mean is
    far from 0), one mixes in values 2^-60 below the rest (the mean's slow
    320-bit path)."""
    R, C = 6, 131072
    rng = np.random.default_rng(10)
    x = np.where(rng.random((R, C)) < 0.5, -1.9921875, 1.9921875).astype(np.float32)
    x[1] *= 2.0 ** 40
    x[2] += 512.0
    x[3, ::3] = 2.0 ** -60
    x[4] = np.where(rng.random(C) < 0.5, 1.9921875, 1.984375).astype(np.float32) * 2.0 ** -100
    xb = W.f32_to_bf16_bits(x)
    print(f"case layernorm long rows R={R} C={C}", flush=True)
    codes, scales, mu, r = sq.w8a8_layernorm_quantize(dev_bf16(xb), None, None, 1e-6)
    torch.cuda.synchronize()
    _check(xb, None, None, 1e-6, codes, scales, mu, r)
