"""Oracle of the quantization steps: K mean, K smoothing, per-block INT8 Q/K
codes and scales, per-block FP8 (E4M3) V codes and scales.

TEST INFRASTRUCTURE.  Part of the CPU oracle; see ``oracle/__init__.py``.

Method, from the pages:
  * Q and K are quantized to low-bit integers so that QK^T runs on the integer
    matrix units (jefxiong.cn "AIGC weekend special 5.10", section 1.2 method
    principle, item (1) SageAttention2++; digipub.cc TurboDiffusion article,
    attention-acceleration paragraph).
  * K is smoothed first: the per-channel mean over tokens is removed, the
    outlier smoothing named in the SageAttention2 title (GVCLab
    Video-Generation-101 systems survey, reference [3]).  Removing one vector
    from every key adds the same constant to every logit of a query row, which
    softmax ignores.
  * V and P may be 8-bit floating point (GVCLab research log 2026-09-02,
    section 5.5 table, SageAttention2 row).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * K mean: mu_c = fl32(sum_n K[n, c] / N) of the EXACT sum, rounded once.
  * K' = fl32(K - mu), binary32, subnormals kept.  Q is not smoothed unless
    asked (quantize_q_smoothed below).
  * Blocks: rows [i*b, min(N, (i+1)*b)) times all d channels, per head.
  * Scale s = fl32(a / 127), a = max |x| over the block; s = 0 when a = 0.
  * Code = clamp(rne(fl32(x / s)), -127, 127); 0 when s = 0.
  * FP8 V: per block of 64 rows a power-of-two scale s_v = 2^e, e the
    smallest integer with max|V| <= 448 * 2^e, at least -127 (s_v = 0 for an
    all-zero block), and code = E4M3FN_rne(V / s_v) (exact division).  A
    power of two is the block-scale form the FP8 matrix instructions apply
    themselves (an E8M0 exponent); for a floating-point code it loses nothing
    against the scale max|V| / 448 but the top fraction of one binade.
"""
from __future__ import annotations

import numpy as np

from . import fp

__all__ = ["kmean_exact", "smooth_k", "block_absmax", "scales_from_absmax", "pow2_scales", "codes_i8",
           "quantize_q", "quantize_k", "quantize_v_fp8", "quantize_q_smoothed"]

# 2^133 turns every bf16 value into an integer (smallest bf16 subnormal is 2^-133)
_BF16_UNIT_EXP = -133


def kmean_exact(k_bits: np.ndarray) -> np.ndarray:
    """Per-channel K mean, mu[c] = fl32(S_c / N) with S_c the exact sum.

    k_bits: uint16 bf16 bits [N, d].  Each value is m * 2^e with an 8-bit
    integer m; the signed m are summed exactly per (channel, exponent) bucket,
    the buckets are combined in Python integers, and the quotient by N is
    rounded once to binary32 (nearest-even)."""
    k_bits = np.asarray(k_bits, np.uint16)
    N, d = k_bits.shape
    neg, m, e = fp.bf16_parts(k_bits)
    sm = np.where(neg == 1, -m, m).astype(np.float64)      # |partial sums| < 2^8 * 2^24 < 2^53: exact
    eb = (e - _BF16_UNIT_EXP).astype(np.int64)              # 0 .. 253
    idx = (np.arange(d, dtype=np.int64)[None, :] * 256 + eb).ravel()
    bucket = np.bincount(idx, weights=sm.ravel(), minlength=d * 256).reshape(d, 256)
    mu = np.empty(d, np.float32)
    for c in range(d):
        total = 0
        for ex in np.nonzero(bucket[c])[0]:
            total += int(bucket[c, ex]) << int(ex)
        # mean = total * 2^-133 / N
        mu[c] = fp.rational_to_f32(total, N << (-_BF16_UNIT_EXP))
    return mu


def smooth_k(k_bits: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """K' = fl32(K - mu) per element (binary32, nearest-even)."""
    return fp.sub_bf16_f32(k_bits, np.asarray(mu, np.float32)[None, :])


def block_absmax(x: np.ndarray, block: int) -> np.ndarray:
    """a_i = max |x| over rows [i*block, min(N, (i+1)*block)) and all channels.
    Exact (a comparison, no arithmetic).  x: float32 [N, d]."""
    x = np.asarray(x, np.float32)
    N = x.shape[0]
    nb = -(-N // block)
    a = np.abs(x).max(axis=1)
    pad = nb * block - N
    if pad:
        a = np.concatenate([a, np.zeros(pad, np.float32)])
    return a.reshape(nb, block).max(axis=1).astype(np.float32)


def scales_from_absmax(a: np.ndarray, qmax: float) -> np.ndarray:
    """s = fl32(a / qmax), correctly rounded; s = 0 where a = 0."""
    a = np.asarray(a, np.float32)
    return fp.div_f32(a, np.float32(qmax)).astype(np.float32)


def codes_i8(x: np.ndarray, s_rows: np.ndarray) -> np.ndarray:
    """code = clamp(rne(fl32(x / s)), -127, 127), 0 where s = 0.

    x: float32 [N, d]; s_rows: float32 [N] (the scale of each row's block)."""
    x = np.asarray(x, np.float32)
    s = np.asarray(s_rows, np.float32)[:, None]
    zero = (s == 0)
    safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
    q = fp.div_f32(x, np.broadcast_to(safe, x.shape))
    # a quotient that overflows binary32 clamps like any other out-of-range one
    q = np.where(np.isinf(q), np.copysign(np.float32(128.0), q), q).astype(np.float32)
    c = np.clip(fp.rne_to_int(q), -127, 127)
    return np.where(np.broadcast_to(zero, x.shape), 0, c).astype(np.int8)


def _rows_scale(s_blocks: np.ndarray, N: int, block: int) -> np.ndarray:
    return np.repeat(np.asarray(s_blocks, np.float32), block)[:N]


def quantize_q(q_bits: np.ndarray, q_block: int):
    """Q [N, d] bf16 bits -> (codes int8 [N, d], scales float32 [nq])."""
    x = (np.asarray(q_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    s = scales_from_absmax(block_absmax(x, q_block), 127.0)
    return codes_i8(x, _rows_scale(s, x.shape[0], q_block)), s


def quantize_k(k_bits: np.ndarray, k_block: int):
    """K [N, d] bf16 bits -> (codes int8 [N, d], scales float32 [nk], mu float32 [d])."""
    mu = kmean_exact(k_bits)
    x = smooth_k(k_bits, mu)
    s = scales_from_absmax(block_absmax(x, k_block), 127.0)
    return codes_i8(x, _rows_scale(s, x.shape[0], k_block)), s, mu


def pow2_scales(a: np.ndarray, qmax: float, emin: int = -127) -> np.ndarray:
    """s = 2^e, e the smallest integer with a <= qmax * 2^e, e >= emin;
    s = 0 where a = 0.  Decided exactly: a = f 2^E with f in [1, 2) and
    qmax = g 2^G with g in [1, 2), a <= qmax 2^e iff e >= E - G when
    f <= g, else e >= E - G + 1."""
    a = np.asarray(a, np.float32).astype(np.float64)
    f, E = np.frexp(a)                          # a = f 2^E, f in [0.5, 1)
    g, G = np.frexp(np.float64(qmax))
    e = np.where(f <= g, E - G, E - G + 1).astype(np.int64)
    e = np.maximum(e, emin)
    return np.where(a == 0, 0.0, np.ldexp(1.0, e)).astype(np.float32)


def quantize_v_fp8(v_bits: np.ndarray, v_block: int = 64):
    """V [N, d] bf16 bits -> (E4M3FN codes uint8 [N, d], power-of-two scales
    float32 [nv])."""
    x = (np.asarray(v_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    s = pow2_scales(block_absmax(x, v_block), fp.E4M3_MAX)
    rows = _rows_scale(s, x.shape[0], v_block)[:, None]
    zero = np.broadcast_to(rows == 0, x.shape)
    safe = np.broadcast_to(np.where(rows == 0, np.float32(1.0), rows).astype(np.float32), x.shape)
    y = fp.div_f32(x, safe)
    codes = fp.e4m3_encode(y)
    return np.where(zero, np.uint8(0), codes).astype(np.uint8), s


def quantize_q_smoothed(q_bits: np.ndarray, q_block: int):
    """Q smoothing, per block of q_block rows: the block's per-channel mean
    mu_b (exact sum rounded once, as the K mean) is removed before the block
    is quantized, and comes back as the logit bias mu_b . K'_j
    (attention.smoothing_bias).  The outlier smoothing of the SageAttention2
    title (GVCLab Video-Generation-101 systems survey, reference [3]) applied
    to Q per block; the pages give no formula, this is the plainest reading
    that keeps QK^T on the integer codes.

    Q' = fl32(Q - mu_b); s = fl32(max|Q'| / 127); codes as quantize_q.  A
    block whose rows are all equal (s = 0: the bias would carry the whole
    logit in units of a zero scale) is quantized plainly instead (mu_b = 0).

    Returns (codes int8 [N, d], scales float32 [nq], mu float32 [nq, d])."""
    q_bits = np.asarray(q_bits, np.uint16)
    N, d = q_bits.shape
    nq = -(-N // q_block)
    x = (q_bits.astype(np.uint32) << 16).view(np.float32)
    codes = np.empty((N, d), np.int8)
    scales = np.empty(nq, np.float32)
    mu = np.zeros((nq, d), np.float32)
    for b in range(nq):
        r0, r1 = b * q_block, min(N, (b + 1) * q_block)
        m = kmean_exact(q_bits[r0:r1])
        xs = smooth_k(q_bits[r0:r1], m)
        sb = scales_from_absmax(np.abs(xs).max().reshape(1), 127.0)[0]
        if sb > 0:
            mu[b] = m
        else:
            xs = x[r0:r1]
            sb = scales_from_absmax(np.abs(xs).max().reshape(1), 127.0)[0]
        scales[b] = sb
        codes[r0:r1] = codes_i8(xs, np.full(r1 - r0, sb, np.float32))
    return codes, scales, mu
