"""Oracle of the W8A8 block-wise INT8 linear layer.

TEST INFRASTRUCTURE.  Part of the CPU oracle; see ``oracle/__init__.py``.

Method, from the pages: the linear layers outside attention quantize both
their weights and their activations to 8-bit integers, block by block with
128x128 blocks, and run the products on the INT8 matrix units (jefxiong.cn
"AIGC weekend special 5.10", section 1.2 item (4), W8A8; digipub.cc
TurboDiffusion article, paragraph on linear-layer quantization).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * The layer is y = x W^T (+ b): x is [M, K] (tokens x in-features), W is
    [N, K] (out-features x in-features), y is [M, N].
  * A block of a [R, C] matrix is rows [128 i, min(R, 128 (i+1))) times
    columns [128 j, 128 (j+1)); C is a multiple of 128.  x and W are blocked
    the same way, so a 128-wide slice j of the reduction axis K meets exactly
    one block of x's row block and one of W's.
  * Scale and code follow the same rule as the attention's Q/K blocks:
    s = fl32(a / 127) with a = max |v| over the block (0 when a = 0), code =
    clamp(rne(fl32(v / s)), -127, 127), 0 when s = 0.
  * y[m, n] = sum_j sx[m // 128, j] * sw[n // 128, j] * D_j[m, n] (+ b[n]),
    D_j[m, n] = sum over k in slice j of cx[m, k] * cw[n, k].  Each D_j is an
    exact integer (|D_j| <= 128 * 127^2 < 2^21); the oracle forms the scaled
    sum in float64.
"""
from __future__ import annotations

import numpy as np

from . import quant

__all__ = ["BLOCK", "quantize_blocks", "linear", "linear_bound"]

BLOCK = 128


def _check_cols(C: int):
    if C % BLOCK:
        raise ValueError(f"the column count ({C}) must be a multiple of {BLOCK}")


def quantize_blocks(x: np.ndarray):
    """x float32 [R, C] (bf16 values widened) -> (codes int8 [R, C],
    scales float32 [ceil(R/128), C/128]), one scale per 128x128 block."""
    x = np.asarray(x, np.float32)
    R, C = x.shape
    _check_cols(C)
    rb, cb = -(-R // BLOCK), C // BLOCK
    codes = np.zeros((R, C), np.int8)
    scales = np.zeros((rb, cb), np.float32)
    for j in range(cb):
        cols = slice(j * BLOCK, (j + 1) * BLOCK)
        # the absmax of a row block over this column slice
        s = quant.scales_from_absmax(quant.block_absmax(x[:, cols], BLOCK), 127.0)
        scales[:, j] = s
        rows_s = np.repeat(s, BLOCK)[:R]
        codes[:, cols] = quant.codes_i8(x[:, cols], rows_s)
    return codes, scales


def _terms(cx, sx, cw, sw):
    """Yields, per 128-wide slice j of K, the float64 matrix
    sx[m//128, j] * sw[n//128, j] * D_j[m, n]."""
    cx = np.asarray(cx, np.int8)
    cw = np.asarray(cw, np.int8)
    M, K = cx.shape
    N, K2 = cw.shape
    if K != K2:
        raise ValueError("x and W disagree on K")
    _check_cols(K)
    sx = np.asarray(sx, np.float32).astype(np.float64)
    sw = np.asarray(sw, np.float32).astype(np.float64)
    rx = np.arange(M) // BLOCK
    rw = np.arange(N) // BLOCK
    for j in range(K // BLOCK):
        cols = slice(j * BLOCK, (j + 1) * BLOCK)
        # integer codes as float64: every product and partial sum is an
        # integer below 2^21, so the library product is exact
        D = cx[:, cols].astype(np.float64) @ cw[:, cols].astype(np.float64).T
        yield (sx[rx, j][:, None] * sw[rw, j][None, :]) * D


def linear(cx, sx, cw, sw, bias=None) -> np.ndarray:
    """The W8A8 layer on quantized operands: float64 [M, N]."""
    cx = np.asarray(cx)
    y = np.zeros((cx.shape[0], np.asarray(cw).shape[0]), np.float64)
    for t in _terms(cx, sx, cw, sw):
        y += t
    if bias is not None:
        y += np.asarray(bias, np.float32).astype(np.float64)[None, :]
    return y


def linear_bound(cx, sx, cw, sw, bias=None) -> np.ndarray:
    """sum_j |sx sw D_j| (+ |b|): the magnitude that bounds the rounding
    error of any evaluation that rounds each slice's term and each partial
    sum once in a given precision (float64 [M, N])."""
    cx = np.asarray(cx)
    a = np.zeros((cx.shape[0], np.asarray(cw).shape[0]), np.float64)
    for t in _terms(cx, sx, cw, sw):
        a += np.abs(t)
    if bias is not None:
        a += np.abs(np.asarray(bias, np.float32).astype(np.float64))[None, :]
    return a
