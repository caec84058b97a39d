"""GPU parity of the W8A8 linear layer: the HIP path (through the C-ABI)
against the CPU oracle (oracle/w8a8.py).

Codes and scales must match bit for bit.  The output y must lie within the
rounding bound of the kernel's fp32 evaluation, derived from its arithmetic:
per 128-wide K slice one rounding of the scale product fl32(sx*sw) and one of
the fused multiply-add into the accumulator, then one for the bias, so with
u = 2^-24 and n slices
    |y - y_oracle| <= (n + 2) u (1 + 1e-3) * sum_j |sx sw D_j| (+ |b|)
(the oracle's float64 sum is exact to far below that); a bf16 output adds
half a bf16 step, at most 2^-9 |y| (2^-8 |y| is allowed).
"""
import math

import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import dev_bf16, host
from oracle import w8a8
from workloads import linear as WL

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def _data(M, N, K, seed, kind="normal", bias=True):
    """x [M, K] and W [N, K] as bf16 bits, bias float32 [N] or None.
    kind "spread": every 128x128 block of x and W scaled by its own 2^e,
    e in [-24, 24], some blocks zero, and planted ties (v = (k + 1/2) s)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K)) / math.sqrt(K)
    if kind == "spread":
        for a in (x, w):
            R = a.shape[0]
            for i in range(-(-R // 128)):
                for j in range(K // 128):
                    blk = a[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
                    if rng.random() < 0.1:
                        blk[:] = 0
                        continue
                    e = int(rng.integers(-24, 25))
                    blk *= 2.0 ** e
                    # absmax exactly 127 * 2^e and a few exact ties
                    blk[0, 0] = 127 * 2.0 ** e
                    blk[-1, 1:5] = np.array([2.5, -3.5, 0.5, 126.5]) * 2.0 ** e
    b = rng.standard_normal(N).astype(np.float32) if bias else None
    return _bits(x), _bits(w), b


def _tol(bound, nkb, y_ref, bf16):
    t = (nkb + 2) * U * (1 + 1e-3) * bound
    if bf16:
        t = t + 2.0 ** -8 * np.abs(y_ref)
    return t


def _check_quant(codes_dev, scales_dev, bits, rows=None):
    """GPU codes/scales (all rows, or the given 128-row blocks) vs the oracle."""
    c_ref, s_ref = w8a8.quantize_blocks(W.bf16_bits_to_f32(bits))
    c, s = host(codes_dev), host(scales_dev)
    if rows is not None:
        r = np.concatenate([np.arange(128 * i, min(c.shape[0], 128 * i + 128)) for i in rows])
        c, s = c[r], s[rows]
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    assert np.array_equal(c, c_ref), "codes differ"
    return c_ref, s_ref


def _check_out(y_dev, y_ref, bound, nkb, bf16, rows=None, cols=None):
    y = host(y_dev.float()).astype(np.float64)
    if rows is not None:
        y = y[np.ix_(rows, cols)]
    tol = _tol(bound, nkb, y_ref, bf16)
    err = np.abs(y - y_ref)
    worst = float((err / np.maximum(tol, 1e-300)).max())
    assert np.all(err <= tol), f"max err/tol {worst:.3g}"
    return worst


@pytest.mark.parametrize("R,C", [(300, 384), (1, 128), (129, 640), (2048, 1280)])
@pytest.mark.parametrize("kind", ["normal", "spread"])
def test_quantize_bit_exact(R, C, kind):
    print(f"case quantize R={R} C={C} kind={kind}", flush=True)
    x, _, _ = _data(R, 1, C, seed=R + C, kind=kind, bias=False)
    codes, scales = sq.w8a8_quantize(dev_bf16(x))
    torch.cuda.synchronize()
    _check_quant(codes, scales, x)


@pytest.mark.parametrize("M,N,K,bias,out", [
    (600, 520, 1280, True, "fp32"),
    (600, 520, 1280, False, "bf16"),
    (1, 1, 128, True, "fp32"),
    (257, 513, 256, True, "fp32"),
    (256, 256, 128, False, "fp32"),
    (300, 300, 8960, True, "fp32"),     # 70 slices: crosses the 64-slice scale staging
    (64, 96, 16512, True, "bf16"),      # 129 slices
    (200, 203, 256, True, "bf16"),      # rows not 16-byte aligned: element-wise tail stores
    (520, 264, 384, False, "bf16"),     # ragged in both, vector stores
])
def test_gemm_parity(M, N, K, bias, out):
    print(f"case gemm M={M} N={N} K={K} bias={bias} out={out}", flush=True)
    xb, wb, b = _data(M, N, K, seed=M * 7 + N * 3 + K, bias=bias)
    xc, xs = sq.w8a8_quantize(dev_bf16(xb))
    wc, ws = sq.w8a8_quantize(dev_bf16(wb))
    bf = out == "bf16"
    y = sq.w8a8_gemm(xc, xs, wc, ws, bias=torch.from_numpy(b).cuda() if bias else None,
                     out_dtype=torch.bfloat16 if bf else torch.float32)
    torch.cuda.synchronize()
    cx, sx = _check_quant(xc, xs, xb)
    cw, sw = _check_quant(wc, ws, wb)
    y_ref = w8a8.linear(cx, sx, cw, sw, b)
    bound = w8a8.linear_bound(cx, sx, cw, sw, b)
    worst = _check_out(y, y_ref, bound, K // 128, bf)
    print(f"  max err/tol {worst:.3g}", flush=True)


def test_gemm_spread_magnitudes():
    M, N, K = 384, 300, 1024
    print(f"case gemm spread M={M} N={N} K={K}", flush=True)
    xb, wb, b = _data(M, N, K, seed=5, kind="spread")
    xc, xs = sq.w8a8_quantize(dev_bf16(xb))
    wc, ws = sq.w8a8_quantize(dev_bf16(wb))
    y = sq.w8a8_gemm(xc, xs, wc, ws, bias=torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    cx, sx = _check_quant(xc, xs, xb)
    cw, sw = _check_quant(wc, ws, wb)
    _check_out(y, w8a8.linear(cx, sx, cw, sw, b), w8a8.linear_bound(cx, sx, cw, sw, b), K // 128, False)


def test_linear_equals_quantize_then_gemm_and_is_deterministic():
    M, N, K = 700, 640, 2560
    print(f"case linear M={M} N={N} K={K}", flush=True)
    xb, wb, b = _data(M, N, K, seed=9)
    X = dev_bf16(xb)
    wc, ws = sq.w8a8_quantize(dev_bf16(wb))
    B = torch.from_numpy(b).cuda()
    y1 = sq.w8a8_linear(X, wc, ws, bias=B)
    xc, xs = sq.w8a8_quantize(X)
    y2 = sq.w8a8_gemm(xc, xs, wc, ws, bias=B)
    y3 = sq.w8a8_linear(X, wc, ws, bias=B)
    yb = sq.w8a8_linear(X, wc, ws, bias=B, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    # the bf16 output is the fp32 result rounded to nearest even
    assert torch.equal(yb, y1.to(torch.bfloat16))


def test_empty_shapes():
    X = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    wc, ws = sq.w8a8_quantize(dev_bf16(_data(64, 1, 256, seed=1, bias=False)[0]))
    y = sq.w8a8_linear(X, wc, ws)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 64)


@pytest.mark.parametrize("name", ["w8a8-qkv-wan14b-480p", "w8a8-out-wan14b-480p", "w8a8-qkv-wan1.3b-480p"])
def test_full_size_sampled(name):
    """Full-size layer as the benchmark runs it (bf16 output, bias); the
    oracle checks the sampled row blocks of x (always holding the ragged last
    one) against sampled row blocks of W (always holding the last)."""
    w = WL.get_linear(name)
    print(f"case full {name} M={w.M} N={w.N} K={w.K}", flush=True)
    x = WL.gen_x(w)
    wt = WL.gen_w(w)
    b = WL.gen_bias(w)
    wc, ws = sq.w8a8_quantize(dev_bf16(wt))
    X = dev_bf16(x)
    y = sq.w8a8_linear(X, wc, ws, bias=torch.from_numpy(b).cuda(), out_dtype=torch.bfloat16)
    xc, xs = sq.w8a8_quantize(X)
    torch.cuda.synchronize()
    del X
    xr = WL.checked_row_blocks(w)
    nbw = -(-w.N // 128)
    rng = np.random.default_rng(w.index)
    wr = np.sort(np.concatenate([rng.choice(nbw - 1, size=5, replace=False), [nbw - 1]]))
    cx, sx = _check_quant(xc, xs, WL.gen_x_blocks(w, xr), rows=xr)
    cw, sw = _check_quant(wc, ws, WL.gen_w_blocks(w, wr), rows=wr)
    rows = np.concatenate([np.arange(128 * i, min(w.M, 128 * i + 128)) for i in xr])
    cols = np.concatenate([np.arange(128 * i, min(w.N, 128 * i + 128)) for i in wr])
    # the oracle's row blocks are the sampled ones, in order: its block index
    # is the position in the sample, which keeps every block's scale aligned
    y_ref = w8a8.linear(cx, sx, cw, sw, b[cols])
    bound = w8a8.linear_bound(cx, sx, cw, sw, b[cols])
    worst = _check_out(y, y_ref, bound, w.K // 128, True, rows=rows, cols=cols)
    print(f"  max err/tol {worst:.3g} over {rows.size} x {cols.size} outputs", flush=True)
