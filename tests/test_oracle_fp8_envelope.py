"""The width of the FP8 ambiguity envelope, pinned against an exact evaluation
of the binary32 logit chain.

On the FP8 P.V path the operand is E4M3(y), y = 448 * exp(s - m_t) (GVCLab
research log 2026-09-02, section 5.5 table, SageAttention2 row: FP8 P.V; the
448 scale and the running max are the readings of the oracle).  An
implementation that evaluates y in binary32 as

    c  = fl32(fl32(sQ * fl32(scale * fl32(log2 e))) * sK)        per key tile
    mn = running max over tiles of fl32(Dmax_tile * c)
    mp = fl32(mn - fl32(log2 448))
    y  = exp2(fl32(D * c - mp))            one fused multiply-add, D exact

can round y to the other E4M3 neighbour where y lies within its own error of
a rounding midpoint.  The oracle widens its check there by a per-row relative
width eps_r = 2^-21 (M_r + 3), M_r the row's largest |logit| in log2 units
(oracle.attention.envelope_width), derived as a bound on that chain's error.
This test pins the width to the chain itself: it evaluates the chain exactly
(float32 products with IEEE rounding, the FMA as the exact float64 value of
product plus addend rounded once to float32, exp2 correctly rounded) on
heavy-tailed workload data and checks, for every element that can round to a
nonzero E4M3 value (y >= 2^-11):

  * the chain's relative deviation from the float64 value stays within
    eps_r - 2^-23, the rest of the width covering v_exp_f32's error (1 ulp);
  * the width is not loose by more than a factor 16 on the worst row, so a
    mistake that inflates it (a dropped factor of M_r, a wrong unit) fails.
"""
import numpy as np

import workloads as W
from oracle import attention as A
from oracle import quant

LOG2E_F32 = np.float32(1.4426950408889634)
LOG2_448_F32 = np.float32(8.80735492205760410)


def _fma_f32(a, b, c):
    """fl32(a * b + c) for float32 arrays: the product of two float32 values is
    exact in float64, and here so is the sum (a few dozen significant bits)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _chain(D, qs_rows, ks_tiles, scale, kv_tile=64):
    """y of every (row, key) by the binary32 chain above; D [R, N] integers."""
    f32 = np.float32
    R, N = D.shape
    nt = N // kv_tile
    sl = f32(f32(scale) * LOG2E_F32)
    cq = (qs_rows.astype(f32) * sl).astype(f32)
    c = (cq[:, None] * ks_tiles.astype(f32)[None, :]).astype(f32)            # [R, nt]
    Dt = D.reshape(R, nt, kv_tile).astype(f32)                                 # exact: |D| < 2^22
    mn = np.maximum.accumulate((Dt.max(axis=2) * c).astype(f32), axis=1)
    mp = (mn - LOG2_448_F32).astype(f32)
    arg = _fma_f32(Dt, np.broadcast_to(c[:, :, None], Dt.shape), np.broadcast_to(-mp[:, :, None], Dt.shape))
    return np.exp2(arg.astype(np.float64)).astype(f32).astype(np.float64).reshape(R, N)


def _exact(D, qs_rows, sk_keys, scale, kv_tile=64):
    """y = 448 exp(s - m_t) in float64, s the oracle's logits, m_t its running max."""
    S = A.logits(D, qs_rows, sk_keys, scale)
    R, N = S.shape
    m = np.maximum.accumulate(S.reshape(R, N // kv_tile, kv_tile).max(axis=2), axis=1)
    return 448.0 * np.exp(S - np.repeat(m, kv_tile, axis=1)), S


def _head(N=4096, stride=8, q_block=None):
    w = W.get("wan14b-480p-fp8")
    q, k, v, _ = W.gen_inputs(w, N=N, B=1, H=1)
    qb = q_block or w.q_block
    qc, qs = quant.quantize_q(q[0, 0], qb)
    kc, ks, _ = quant.quantize_k(k[0, 0], 64)
    rows = np.arange(0, N, stride)
    D = A.int_scores(qc[rows], kc)
    return w, D, qs[rows // qb].astype(np.float64), ks


def _ratios(q_block=None):
    w, D, qs_rows, ks = _head(q_block=q_block)
    y_chain = _chain(D, qs_rows, ks, w.scale)
    y_ref, S = _exact(D, qs_rows, np.repeat(ks.astype(np.float64), 64)[:D.shape[1]], w.scale)
    rel = np.where(y_ref >= 2.0 ** -11, np.abs(y_chain - y_ref) / y_ref, 0.0)
    eps = A.envelope_width(np.abs(S).max(axis=1) / np.log(2.0))
    return rel.max(axis=1), eps


def test_chain_error_within_width():
    worst, eps = _ratios()
    assert np.all(worst <= eps - 2.0 ** -23), float((worst / eps).max())


def test_chain_error_within_width_per_row_q_scales():
    worst, eps = _ratios(q_block=1)
    assert np.all(worst <= eps - 2.0 ** -23), float((worst / eps).max())


def test_width_not_loose():
    worst, eps = _ratios()
    assert (worst / eps).max() >= 1.0 / 16.0, float((worst / eps).max())


def test_width_formula():
    assert A.envelope_width(0.0) == 3.0 * 2.0 ** -21
    assert np.isclose(A.envelope_width(253.0), 2.0 ** -13)
