"""GPU parity of RMSNorm fused with the W8A8 block quantization
(sqattn_w8a8_rmsnorm_quantize / sqattn_w8a8_linear_rmsnorm) against
oracle/norm.py: inverse RMS, codes and scales bit for bit; the fused linear
equals quantize + gemm bit for bit."""
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
    x = rng.standard_normal((R, C)) * rng.uniform(0.05, 20, (R, 1))
    if kind == "spread":
        e = rng.integers(-60, 61, R)
        x = x * np.ldexp(1.0, e)[:, None]
        x[0] = 0.0                                            # zero row: r = 1/sqrt(eps)
        if R > 2:
            x[1, : C // 2] = rng.standard_normal(C // 2) * 1e-39   # subnormals beside normal values
            x[2] = rng.standard_normal(C) * 1e37 * 3               # mean square overflows: r = 0
        x[-1, ::7] = 0.0
    return W.f32_to_bf16_bits(x.astype(np.float32))


def _check(xb, gamma, eps, codes, scales, r):
    c_ref, s_ref, r_ref = norm.rmsnorm_quantize(xb, gamma, eps)
    assert np.array_equal(host(r).view(np.uint32), r_ref.view(np.uint32)), "inverse RMS differs"
    assert np.array_equal(host(scales).view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    assert np.array_equal(host(codes), c_ref), "codes differ"


@pytest.mark.parametrize("R,C", [(300, 384), (1, 128), (129, 640), (1000, 5120)])
@pytest.mark.parametrize("kind", ["normal", "spread"])
@pytest.mark.parametrize("affine", [False, True])
def test_rmsnorm_quantize_bit_exact(R, C, kind, affine):
    print(f"case rmsnorm R={R} C={C} kind={kind} gamma={affine}", flush=True)
    xb = _rows(R, C, seed=R + C + (7 if affine else 0), kind=kind)
    g = (np.random.default_rng(C).standard_normal(C) * 0.3 + 1).astype(np.float32) if affine else None
    eps = 1e-6
    codes, scales, r = sq.w8a8_rmsnorm_quantize(dev_bf16(xb), None if g is None else torch.from_numpy(g).cuda(), eps)
    torch.cuda.synchronize()
    _check(xb, g, eps, codes, scales, r)


def test_linear_rmsnorm_equals_quantize_then_gemm():
    M, N, K = 700, 640, 2560
    rng = np.random.default_rng(3)
    X = dev_bf16(_rows(M, K, seed=4, kind="normal"))
    wb = W.f32_to_bf16_bits((rng.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32))
    wc, ws = sq.w8a8_quantize(dev_bf16(wb))
    g = torch.from_numpy((rng.standard_normal(K) * 0.2 + 1).astype(np.float32)).cuda()
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).cuda()
    y1 = sq.w8a8_linear_rmsnorm(X, wc, ws, gamma=g, eps=1e-6, bias=b, out_dtype=torch.bfloat16)
    xc, xs, _ = sq.w8a8_rmsnorm_quantize(X, g, 1e-6)
    y2 = sq.w8a8_gemm(xc, xs, wc, ws, bias=b, out_dtype=torch.bfloat16)
    y3 = sq.w8a8_linear_rmsnorm(X, wc, ws, gamma=g, eps=1e-6, bias=b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_full_size_qkv_input():
    """The 14B QKV projection input (32760 x 5120): inverse RMS of every row,
    codes and scales of the sampled row blocks."""
    w = WL.get_linear("w8a8-qkv-wan14b-480p")
    print(f"case rmsnorm full M={w.M} K={w.K}", flush=True)
    x = WL.gen_x(w)
    g = (np.random.default_rng(5).standard_normal(w.K) * 0.2 + 1).astype(np.float32)
    codes, scales, r = sq.w8a8_rmsnorm_quantize(dev_bf16(x), torch.from_numpy(g).cuda(), 1e-6)
    torch.cuda.synchronize()
    _, r_ref = norm.rms_inverse(x, 1e-6)
    assert np.array_equal(host(r).view(np.uint32), r_ref.view(np.uint32))
    blocks = WL.checked_row_blocks(w)
    rows = np.concatenate([np.arange(128 * i, min(w.M, 128 * i + 128)) for i in blocks])
    c_ref, s_ref, _ = norm.rmsnorm_quantize(x[rows], g, 1e-6)
    assert np.array_equal(host(scales)[blocks].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(codes)[rows], c_ref)


def test_long_rows_fill_the_fast_window():
    """Rows of 131072 values of the largest significand at one exponent: every
    square sits at the top of the 64-bit window, which must be emptied into
    the full accumulator before it overflows."""
    R, C = 8, 131072
    rng = np.random.default_rng(9)
    x = np.where(rng.random((R, C)) < 0.5, -1.9921875, 1.9921875).astype(np.float32)
    x[1] *= 2.0 ** 40
    x[2, ::3] = 2.0 ** -20          # squares far below the window's top
    xb = W.f32_to_bf16_bits(x)
    codes, scales, r = sq.w8a8_rmsnorm_quantize(dev_bf16(xb), None, 1e-6)
    torch.cuda.synchronize()
    _check(xb, None, 1e-6, codes, scales, r)


def test_mean_square_next_to_a_midpoint():
    """Rows whose kept squares leave the mean square just under a binary32
    midpoint and whose squares 2^150 and 2^300 below the largest decide the
    rounding: tie (to even), above and below, settled one or two levels
    down.  Each row's two candidates give different inverse RMS values."""
    import norm_cases as NC
    rows = [NC.mean_square_row(kind, seed=11 * i) for i, kind in enumerate(NC.KINDS)]
    x1 = np.stack([b for b, _, _, _ in rows])
    want = np.array([w for _, _, _, w in rows], np.float32)
    # each row also tiled 4 times (1024 columns, same mean square, every
    # level sum and gap scaled by 4: the same decisions, over two loads a lane)
    for xb in (x1, np.tile(x1, (1, 4))):
        print(f"case midpoint rows R={xb.shape[0]} C={xb.shape[1]}", flush=True)
        codes, scales, r = sq.w8a8_rmsnorm_quantize(dev_bf16(xb), None, NC.EPS)
        torch.cuda.synchronize()
        _check(xb, None, NC.EPS, codes, scales, r)
        assert np.array_equal(host(r), np.float32(1) / np.sqrt(want + np.float32(NC.EPS)))
