"""Oracle of the RMSNorm that precedes the W8A8 projections, fused with their
INT8 block quantization.

TEST INFRASTRUCTURE.  Part of the CPU oracle; see ``oracle/__init__.py``.

Method, from the pages: TurboDiffusion rewrites LayerNorm and RMSNorm as
custom kernels for speed (digipub.cc TurboDiffusion article, paragraph on
other optimizations), and quantizes the inputs of its linear layers to INT8
in 128x128 blocks (same article, linear-layer quantization paragraph).  The
normalization here feeds that quantization directly.

Readings (the pages give no formula; this is the usual RMSNorm with every
rounding fixed so that a quantization decision never depends on a summation
order):
  * For a row x of K bf16 values: S = sum_k x_k^2 exactly, mu2 =
    fl32(S / K) (the exact quotient rounded once, nearest-even).
  * r = fl32(1 / fl32(sqrt(fl32(mu2 + eps)))): three binary32 operations,
    each correctly rounded; eps > 0 is a binary32 number.
  * y_k = fl32(fl32(x_k * r) * gamma_k) (gamma binary32 [K]; without gamma
    y_k = fl32(x_k * r)).
  * The codes and scales are those of the W8A8 rule applied to the binary32
    y (oracle.w8a8.quantize_blocks): no bf16 round trip in between.
  * LayerNorm (same passage; the normalization in front of a DiT block's
    QKV projection, with its modulation folded into gamma and beta), two-pass
    and order-independent: mu = fl32(S / K) with S = sum_k x_k exact;
    d_k = fl32(x_k - mu); var = fl32(sum_k d_k^2 / K) from the exact sum of
    the binary32 squares; r = fl32(1 / fl32(sqrt(fl32(var + eps))));
    y_k = fl32(fl32(d_k * r) * gamma_k) and then fl32(y_k + beta_k) (each
    factor optional).  Inputs are finite.
  * In front of attention (q/k normalization over each token's H*d features,
    ``qk_rmsnorm``) y is stored in bf16, nearest-even, as the attention
    inputs are; the attention oracle then takes those bf16 tensors.
"""
from __future__ import annotations

import numpy as np

from . import fp, w8a8

__all__ = ["sum_squares_exact", "rms_inverse", "rmsnorm", "rmsnorm_quantize", "qk_rmsnorm", "sum_exact",
           "sum_squares_f32_exact", "layernorm_stats", "layernorm", "layernorm_quantize"]

# every bf16 square is an integer multiple of 2^-266 (smallest subnormal^2)
_UNIT_EXP = -266


def sum_squares_exact(x_bits: np.ndarray) -> list:
    """S_r = sum_k x_rk^2 as exact integers in units of 2^-266, per row.

    x_bits: uint16 bf16 bits [R, K].  A value with biased exponent E and
    significand M (hidden bit included) squares to M^2 * 2^(2 max(E,1) - 2)
    units; the M^2 are summed per exponent bucket (exact in float64: below
    2^36) and the buckets combined in Python integers."""
    b = np.asarray(x_bits, np.uint16).astype(np.int64)
    E = (b >> 7) & 0xFF
    M = (b & 0x7F) | np.where(E > 0, 0x80, 0)
    e2 = 2 * np.maximum(E, 1) - 2                       # 0 .. 506
    R = b.shape[0]
    nb = 2 * 255
    idx = (np.arange(R, dtype=np.int64)[:, None] * nb + e2).ravel()
    buckets = np.bincount(idx, weights=(M * M).astype(np.float64).ravel(), minlength=R * nb).reshape(R, nb)
    out = []
    for r in range(R):
        s = 0
        for e in np.nonzero(buckets[r])[0]:
            s += int(buckets[r, e]) << int(e)
        out.append(s)
    return out


def rms_inverse(x_bits: np.ndarray, eps: float):
    """(mu2, r) per row, float32 [R] each."""
    x_bits = np.asarray(x_bits, np.uint16)
    K = x_bits.shape[1]
    S = sum_squares_exact(x_bits)
    mu2 = np.array([fp.rational_to_f32(s, K << -_UNIT_EXP) for s in S], np.float32)
    with np.errstate(divide="ignore"):
        r = np.float32(1.0) / np.sqrt(mu2 + np.float32(eps))
    return mu2, r.astype(np.float32)


def rmsnorm(x_bits: np.ndarray, gamma, eps: float):
    """y float32 [R, K] and r float32 [R]."""
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    _, r = rms_inverse(x_bits, eps)
    y = (x * r[:, None]).astype(np.float32)
    if gamma is not None:
        y = (y * np.asarray(gamma, np.float32)[None, :]).astype(np.float32)
    return y, r


def rmsnorm_quantize(x_bits: np.ndarray, gamma, eps: float):
    """(codes int8 [R, K], scales float32 [ceil(R/128), K/128], r float32 [R])."""
    y, r = rmsnorm(x_bits, gamma, eps)
    codes, scales = w8a8.quantize_blocks(y)
    return codes, scales, r


def qk_rmsnorm(x_bits: np.ndarray, gamma, eps: float) -> np.ndarray:
    """The per-token q (or k) normalization in front of attention, stored in
    bf16 as the attention inputs are: for x [B, H, N, d] (bf16 bits) each
    token (b, n) is the row of its H*d values (head-major), normalized as
    ``rmsnorm`` with gamma [H*d] (or None) and rounded to bf16 (nearest even).
    Returns bf16 bits [B, H, N, d]."""
    x = np.asarray(x_bits, np.uint16)
    B, H, N, d = x.shape
    rows = x.transpose(0, 2, 1, 3).reshape(B * N, H * d)
    y, _ = rmsnorm(rows, gamma, eps)
    yb = fp.f32_to_bf16(y)
    return np.ascontiguousarray(yb.reshape(B, N, H, d).transpose(0, 2, 1, 3))


# every binary32 square is an integer multiple of 2^-298; with the
# significands normalised (fp.f32_parts: subnormals shifted up, exponents down
# to -172) the bucket exponents are counted from 2^-344
_F32_SQ_UNIT = -344


def sum_exact(x_bits: np.ndarray) -> list:
    """S_r = sum_k x_rk exactly, as signed integers in units of 2^-133 (the
    smallest bf16 subnormal), per row: signed significands summed per exponent
    bucket (exact in float64: below 2^29), buckets combined in Python ints."""
    b = np.asarray(x_bits, np.uint16).astype(np.int64)
    E = (b >> 7) & 0xFF
    M = (b & 0x7F) | np.where(E > 0, 0x80, 0)
    sM = np.where((b >> 15) == 1, -M, M)
    sh = np.maximum(E, 1) - 1                                  # value = sM * 2^(sh - 133)
    R = b.shape[0]
    idx = (np.arange(R, dtype=np.int64)[:, None] * 256 + sh).ravel()
    buckets = np.bincount(idx, weights=sM.astype(np.float64).ravel(), minlength=R * 256).reshape(R, 256)
    out = []
    for r in range(R):
        s = 0
        for e in np.nonzero(buckets[r])[0]:
            s += int(buckets[r, e]) << int(e)
        out.append(s)
    return out


def sum_squares_f32_exact(d: np.ndarray) -> list:
    """sum_k d_rk^2 exactly for binary32 d [R, K], as integers in units of
    2^-344, per row.  d = m 2^e (fp.f32_parts) squares to m^2 2^(2e); m is
    split as mh 2^12 + ml so that the three partial products summed per
    exponent bucket stay exact in float64."""
    neg, m, e = fp.f32_parts(np.asarray(d, np.float32))
    mh, ml = m >> 12, m & 0xFFF
    e2 = 2 * e - _F32_SQ_UNIT                                  # >= 0
    assert e2.size == 0 or e2.min() >= 0
    R = d.shape[0]
    nb = int(e2.max()) + 1 if e2.size else 1
    idx = (np.arange(R, dtype=np.int64)[:, None] * nb + e2).ravel()
    parts = []
    for w in (mh * mh, 2 * mh * ml, ml * ml):
        parts.append(np.bincount(idx, weights=w.astype(np.float64).ravel(), minlength=R * nb).reshape(R, nb))
    out = []
    for r in range(R):
        s = 0
        for k in np.nonzero(parts[0][r] + parts[1][r] + parts[2][r])[0]:
            s += (int(parts[0][r, k]) << (int(k) + 24)) + (int(parts[1][r, k]) << (int(k) + 12)) \
                + (int(parts[2][r, k]) << int(k))
        out.append(s)
    return out


def layernorm_stats(x_bits: np.ndarray, eps: float):
    """(mu, var, r) per row, float32 [R] each."""
    x_bits = np.asarray(x_bits, np.uint16)
    K = x_bits.shape[1]
    mu = np.array([fp.rational_to_f32(s, K << 133) for s in sum_exact(x_bits)], np.float32)
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    d = (x - mu[:, None]).astype(np.float32)
    var = np.array([fp.rational_to_f32(s, K << -_F32_SQ_UNIT) for s in sum_squares_f32_exact(d)], np.float32)
    with np.errstate(divide="ignore"):
        r = (np.float32(1.0) / np.sqrt(var + np.float32(eps))).astype(np.float32)
    return mu, var, r


def layernorm(x_bits: np.ndarray, gamma, beta, eps: float):
    """y float32 [R, K], mu and r float32 [R]."""
    mu, _, r = layernorm_stats(x_bits, eps)
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    d = (x - mu[:, None]).astype(np.float32)
    y = (d * r[:, None]).astype(np.float32)
    if gamma is not None:
        y = (y * np.asarray(gamma, np.float32)[None, :]).astype(np.float32)
    if beta is not None:
        y = (y + np.asarray(beta, np.float32)[None, :]).astype(np.float32)
    return y, mu, r


def layernorm_quantize(x_bits: np.ndarray, gamma, beta, eps: float):
    """(codes int8 [R, K], scales [ceil(R/128), K/128], mu [R], r [R])."""
    y, mu, r = layernorm(x_bits, gamma, beta, eps)
    codes, scales = w8a8.quantize_blocks(y)
    return codes, scales, mu, r
