"""Oracle of the attention step on quantized operands.

TEST INFRASTRUCTURE.  Part of the CPU oracle; see ``oracle/__init__.py``.

Method, from the pages: QK^T is taken on the low-bit Q and K codes (integer
matrix units), then softmax, then P.V in 16-bit or FP8 (jefxiong.cn "AIGC
weekend special 5.10", section 1.2 item (1); GVCLab research log 2026-09-02,
section 5.5 table, SageAttention2 row).  The tiling with a running max and a
running sum is the FlashAttention lineage the same digest names as the
baseline (section 1.1 and the paper timeline).

Readings where the pages are silent:
  * logits s_rj = D_rj * sQ[r // bq] * sK[j // bk] * scale with D the exact
    integer dot product of the codes; the softmax scale is applied here, not
    folded into Q before quantization; attention is non-causal over all N keys.
  * 16-bit P.V: exact two-pass softmax in float64 with V the exact bf16 values
    (the kernel's bf16 rounding of P is not mirrored; it sits far inside the
    output tolerance).
  * Block-sparse attention (the kernel half of the "sparse + low-bit"
    composition, digipub.cc TurboDiffusion article, SLA paragraph; GVCLab
    Video-Generation-101 systems survey, SpargeAttention row): an optional
    block mask with one entry per (128-row query block, 64-key tile); keys of
    a zero entry get zero weight in that block's rows (logit -inf).  A row
    whose blocks are all zero has no softmax; its output is defined as 0.
  * FP8 P.V: the kernel's online schedule is mirrored.  Keys are taken in tiles
    of ``kv_tile`` in ascending order with running max m_t; P~_j =
    exp(s_j - m_t(j)) in (0, 1]; the FP8 operand is E4M3(448 * P~_j); the row
    sum accumulates the unrounded P~; V enters as s_v * decode(code_v).
    Elements whose 448*P~ lies within ``eps_rel`` (relative) of an E4M3
    rounding midpoint may legitimately round either way in the kernel's
    binary32 arithmetic; the possible effect of each is summed into a
    per-element envelope E.  The default width is per row,
    eps_r = 2^-21 * (M_r + 3), M_r the row's largest |logit| in log2 units,
    a bound on the relative error of 448*P~ computed in binary32 as
      c  = fl32(fl32(sQ * fl32(scale * fl32(log2 e))) * sK)   (per tile)
      mn = running max of fl32(Dmax_tile * c),  mp = fl32(mn - fl32(log2 448))
      y  = exp2(fl32(D * c - mp))          (one fused multiply-add, D exact)
    Only elements with y >= 2^-11 can round to a nonzero E4M3 value, so
    |arg| <= 11 there.  With u = 2^-24: c is off by <= 4u relative (|D c| <=
    M_r: 4u M_r), the running max by <= 5u M_r, mp's rounding adds
    u (M_r + 9), fl32(log2 448) 8u, the FMA 11u, so the exponent argument is
    off by <= u (10 M_r + 28); times ln 2, plus 2u for v_exp_f32 (1 ulp),
    the relative error of y is <= u (6.94 M_r + 21.4) < 2^-21 (M_r + 3).
    tests/test_oracle_fp8_envelope.py checks this bound against an exact
    evaluation of that binary32 chain on heavy-tailed data.
  * Q smoothing (optional, quant.quantize_q_smoothed): the logits gain the
    bias mu_b . K'_j of the row's Q block b, exact (float64 products of the
    binary32 mean and smoothed K), times the softmax scale.  On the FP8 path
    a kernel that takes the bias in units of sQ sK as a binary32 dot product
    (16 FMA chains of 8 terms, summed pairwise) divided by fl32(sQ sK)
    (correctly rounded), and adds it to the converted integer score with one
    rounding, is off by at most 14 u A_j / (sQ sK) units (A_j =
    sum_c |mu_c K'_jc|) plus u |S + bias|; times c that is at most
    u (14 scale log2(e) A_j + M_r) in log2 units, and the envelope widens by
    ln 2 u (16 scale log2(e) max_j A_j + 2 M_r) relative (smoothing_width).
    The 16-bit path's tolerance covers a bias rounded to an integer.
"""
from __future__ import annotations

import numpy as np

from . import fp

__all__ = ["int_scores", "logits", "softmax_pv", "attention_fp64", "attend_bf16",
           "attend_fp8", "e4m3_round_f64", "envelope_width", "MASK_Q", "MASK_K", "key_mask",
           "smoothing_bias", "smoothing_width"]

MASK_Q = 128   # query rows per block-mask row
MASK_K = 64    # keys per block-mask column


def key_mask(block_mask, rows, N) -> np.ndarray:
    """Per-(row, key) keep flags [R, N] of a block mask [ceil(N/128), ceil(N/64)]."""
    bm = np.asarray(block_mask) != 0
    rows = np.asarray(rows, np.int64)
    return bm[rows // MASK_Q][:, np.arange(N) // MASK_K]


def int_scores(q_codes: np.ndarray, k_codes: np.ndarray) -> np.ndarray:
    """D = q_codes @ k_codes^T as exact integers held in float64.

    |D| <= d * 127^2 < 2^53, and every partial sum is an integer of smaller
    magnitude, so float64 BLAS returns the exact value in any summation order."""
    return np.asarray(q_codes, np.float64) @ np.asarray(k_codes, np.float64).T


def logits(D: np.ndarray, sq_rows: np.ndarray, sk_keys: np.ndarray, scale: float) -> np.ndarray:
    """s = D * sQ(row) * sK(key) * scale, float64."""
    return (D * np.asarray(sq_rows, np.float64)[:, None]
            * np.asarray(sk_keys, np.float64)[None, :] * float(scale))


def softmax_pv(S: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Two-pass softmax and product: O = sum_j e^(s_j - m) v_j / sum_j e^(s_j - m)."""
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    return (P @ np.asarray(V, np.float64)) / P.sum(axis=1, keepdims=True)


def attention_fp64(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Unquantized attention softmax(Q K^T * scale) V in float64 (the textbook
    operation the quantized path approximates)."""
    S = (np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T) * float(scale)
    return softmax_pv(S, V)


def smoothing_bias(q_mean, k_smooth, rows, q_block) -> np.ndarray:
    """Delta S [R, N] = mu_b(r) . K'_j in float64: q_mean float32 [nq, d] (zero
    rows for blocks quantized plainly), k_smooth float32 K' [N, d]."""
    rows = np.asarray(rows, np.int64)
    mu = np.asarray(q_mean, np.float32).astype(np.float64)[rows // q_block]
    return mu @ np.asarray(k_smooth, np.float32).astype(np.float64).T


def smoothing_width(q_mean, k_smooth, rows, q_block, scale, max_abs_logit_log2) -> np.ndarray:
    """Extra relative FP8 envelope width per row [R, 1] for the Q-smoothing
    bias computed as the module notes describe: ln 2 u (16 scale log2(e)
    max_j A_j + 2 M_r), A_j = sum_c |mu_c K'_jc| of the row's block."""
    rows = np.asarray(rows, np.int64)
    u = 2.0 ** -24
    mu = np.abs(np.asarray(q_mean, np.float32).astype(np.float64)[rows // q_block])
    A = (mu @ np.abs(np.asarray(k_smooth, np.float32).astype(np.float64)).T).max(axis=1, keepdims=True)
    M = np.asarray(max_abs_logit_log2, np.float64)
    return np.log(2.0) * u * (16.0 * scale * np.log2(np.e) * A + 2.0 * M)


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attend_bf16(q_codes, q_scale, k_codes, k_scale, v_bits, rows, q_block, k_block, scale,
                chunk: int = 256, block_mask=None, q_mean=None, k_smooth=None) -> np.ndarray:
    """Output rows O[rows] (float64 [R, d]) of the 16-bit P.V path for one head
    (block_mask: optional [ceil(N/128), ceil(N/64)], nonzero = computed;
    q_mean/k_smooth: the Q-smoothing bias, see smoothing_bias)."""
    rows = np.asarray(rows, np.int64)
    N = k_codes.shape[0]
    sk = np.repeat(np.asarray(k_scale, np.float64), k_block)[:N]
    V = _bf16_to_f64(v_bits)
    out = np.empty((rows.size, V.shape[1]), np.float64)
    for i in range(0, rows.size, chunk):
        r = rows[i:i + chunk]
        D = int_scores(q_codes[r], k_codes)
        S = logits(D, np.asarray(q_scale, np.float64)[r // q_block], sk, scale)
        if q_mean is not None:
            S = S + smoothing_bias(q_mean, k_smooth, r, q_block) * scale
        if block_mask is None:
            out[i:i + chunk] = softmax_pv(S, V)
            continue
        keep = key_mask(block_mask, r, N)
        live = keep.any(axis=1)
        o = np.zeros((r.size, V.shape[1]), np.float64)
        if live.any():
            o[live] = softmax_pv(np.where(keep[live], S[live], -np.inf), V)
        out[i:i + chunk] = o
    return out


def envelope_width(max_abs_logit_log2):
    """Relative width eps_r = 2^-21 (M_r + 3) of the FP8 ambiguity band for a
    row whose largest |logit| is M_r (log2 units); see the module docstring."""
    return 2.0 ** -21 * (3.0 + np.asarray(max_abs_logit_log2, np.float64))


def e4m3_round_f64(y: np.ndarray):
    """Nearest-even E4M3FN rounding of non-negative float64 values.

    Returns (rounded value, quantum, position of y in units of the quantum);
    saturates at 448."""
    y = np.asarray(y, np.float64)
    _, ex = np.frexp(y)                     # y = f * 2^ex, f in [0.5, 1)
    k = ex - 1                              # binade: 2^k <= y < 2^(k+1)
    qe = np.maximum(k - 3, -9)
    quantum = np.ldexp(1.0, qe)
    c = y / quantum                         # exact: division by a power of two
    r = np.rint(c) * quantum                # rint: round half to even
    r = np.where(y == 0, 0.0, r)
    return np.minimum(r, fp.E4M3_MAX), quantum, c


def attend_fp8(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, rows, q_block, k_block,
               scale, v_block: int = 64, kv_tile: int = 64, eps_rel: float | None = None,
               round_p=None, chunk: int = 128, block_mask=None, q_mean=None, k_smooth=None):
    """FP8 P.V path for one head; returns (O [R, d], E [R, d], hits).

    ``round_p`` maps 448*P~ to the FP8 operand value (default: E4M3 rounding;
    the identity turns the mirror into the exact softmax, a self-check).
    With ``block_mask`` the running max is taken over kept keys only (tiles
    without a kept key leave it unchanged) and dropped keys have P~ = 0."""
    rows = np.asarray(rows, np.int64)
    N = k_codes.shape[0]
    sk = np.repeat(np.asarray(k_scale, np.float64), k_block)[:N]
    sv = np.repeat(np.asarray(v_scale, np.float64), v_block)[:N]
    Vh = fp.e4m3_decode(v_codes) * sv[:, None]           # dequantized V
    absV = np.abs(Vh)
    nt = -(-N // kv_tile)
    pad = nt * kv_tile - N
    O = np.empty((rows.size, Vh.shape[1]), np.float64)
    E = np.zeros_like(O)
    hits = 0
    for i in range(0, rows.size, chunk):
        r = rows[i:i + chunk]
        S = logits(int_scores(q_codes[r], k_codes), np.asarray(q_scale, np.float64)[r // q_block],
                   sk, scale)
        if q_mean is not None:
            S = S + smoothing_bias(q_mean, k_smooth, r, q_block) * scale
        keep = np.ones(S.shape, bool) if block_mask is None else key_mask(block_mask, r, N)
        live = keep.any(axis=1, keepdims=True)
        Sk = np.where(keep, S, -np.inf)
        Sp = np.pad(Sk, ((0, 0), (0, pad)), constant_values=-np.inf)
        tile_max = Sp.reshape(r.size, nt, kv_tile).max(axis=2)
        m_run = np.maximum.accumulate(tile_max, axis=1)          # m_t
        m_key = np.repeat(m_run, kv_tile, axis=1)[:, :N]         # m_t(j)
        m_T = np.where(live, m_run[:, -1:], 0.0)
        m_key = np.where(keep, m_key, 0.0)
        Pt = np.where(keep, np.exp(np.where(keep, S, 0.0) - m_key), 0.0)   # P~ in (0, 1], 0 if dropped
        y = 448.0 * Pt
        if round_p is None:
            yr, quantum, c = e4m3_round_f64(y)
        else:
            yr = round_p(y)
        w = np.where(keep, np.exp(m_key - m_T), 0.0)             # e^(m_t(j) - m_T)
        l = (w * Pt).sum(axis=1, keepdims=True)
        num = (w * yr / 448.0) @ Vh
        O[i:i + chunk] = np.where(live, num / np.where(live, l, 1.0), 0.0)
        if round_p is None:
            if eps_rel is None:
                # the largest |logit| among the keys the kernel evaluates (kept keys)
                M = np.where(keep, np.abs(S), 0.0).max(axis=1, keepdims=True) / np.log(2.0)
                eps = envelope_width(M)
                if q_mean is not None:
                    eps = eps + smoothing_width(q_mean, k_smooth, r, q_block, scale, M)
            else:
                eps = eps_rel
            frac = c - np.floor(c)
            amb = (np.abs(frac - 0.5) * quantum <= eps * y) & (y > 0)
            if amb.any():
                lo = np.floor(c) * quantum
                hi = np.minimum((np.floor(c) + 1.0) * quantum, fp.E4M3_MAX)
                dP = np.where(amb, (hi - lo) / 448.0 * w, 0.0)
                E[i:i + chunk] = np.where(live, (dP @ absV) / np.where(live, l, 1.0), 0.0)
                hits += int(amb.sum())
    return O, E, hits
