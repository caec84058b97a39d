"""Pins of the oracle's attention step.

Checked against torch's CPU scaled_dot_product_attention in float64 (an
independent library routine), Python-integer brute force for the integer
scores, a per-tile loop of the online-softmax recurrence written step by step
(for the FP8 mirror, whose production form is vectorized), closed forms
(N = 1, Q = 0, constant V, one dominant logit) and invariants (softmax rows sum
to 1, K mean-subtraction leaves exact attention unchanged, joint key/value
permutation invariance, whole-block permutations of the quantized pipeline).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import fp, quant
import workloads as W


def _sdpa(Q, K, V, scale):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), scale=scale)[0, 0].numpy()


def test_attention_fp64_matches_torch_sdpa():
    rng = np.random.default_rng(0)
    for (R, N, d) in [(5, 7, 3), (33, 130, 64), (64, 257, 128)]:
        Q, K, V = rng.standard_normal((R, d)) * 2, rng.standard_normal((N, d)), rng.standard_normal((N, d))
        sc = 1 / math.sqrt(d)
        np.testing.assert_allclose(A.attention_fp64(Q, K, V, sc), _sdpa(Q, K, V, sc), rtol=0, atol=1e-13)


def test_softmax_rows_sum_to_one_and_closed_forms():
    rng = np.random.default_rng(1)
    N = 40
    S = rng.standard_normal((6, N)) * 10
    P = A.softmax_pv(S, np.eye(N))                 # V = I returns the weights themselves
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-15)
    assert (P >= 0).all()
    # N = 1: output is the single value row
    V1 = rng.standard_normal((1, 8))
    np.testing.assert_allclose(A.softmax_pv(rng.standard_normal((3, 1)), V1), np.repeat(V1, 3, 0), atol=1e-15)
    # all-equal logits (Q = 0): output is the mean of V
    V = rng.standard_normal((N, 8))
    np.testing.assert_allclose(A.attention_fp64(np.zeros((2, 4)), rng.standard_normal((N, 4)), V, 1.0),
                               np.repeat(V.mean(0, keepdims=True), 2, 0), atol=1e-14)
    # constant V: constant output
    Vc = np.tile(rng.standard_normal((1, 8)), (N, 1))
    np.testing.assert_allclose(A.softmax_pv(S, Vc), np.repeat(Vc[:1], 6, 0), atol=1e-14)
    # one dominant logit selects its value row
    S2 = np.zeros((1, N))
    S2[0, 17] = 800.0
    np.testing.assert_allclose(A.softmax_pv(S2, V), V[17:18], atol=1e-300)


def test_k_mean_subtraction_invariance_and_permutation():
    rng = np.random.default_rng(2)
    Q, K, V = rng.standard_normal((16, 32)), rng.standard_normal((90, 32)) + 3, rng.standard_normal((90, 32))
    O = A.attention_fp64(Q, K, V, 0.2)
    np.testing.assert_allclose(A.attention_fp64(Q, K - K.mean(0), V, 0.2), O, atol=1e-12)
    p = rng.permutation(90)
    np.testing.assert_allclose(A.attention_fp64(Q, K[p], V[p], 0.2), O, atol=1e-13)


def test_int_scores_exact():
    rng = np.random.default_rng(3)
    qc = rng.integers(-127, 128, (9, 128)).astype(np.int8)
    kc = rng.integers(-127, 128, (11, 128)).astype(np.int8)
    qc[0] = 127
    kc[0] = -127
    D = A.int_scores(qc, kc)
    for i in range(9):
        for j in range(11):
            assert D[i, j] == sum(int(a) * int(b) for a, b in zip(qc[i], kc[j]))
    assert D[0, 0] == -128 * 127 * 127


def _head(N=300, d=64, seed=4, dist="normal"):
    w = W.Workload(99, "t", 1, 1, N, d, 64, 64, dist, "bf16", 0)
    rng = np.random.default_rng(seed)
    raw = (lambda s: rng.standard_normal(s)) if dist == "normal" else (lambda s: rng.standard_t(3, s))
    q = W.f32_to_bf16_bits(raw((N, d)).astype(np.float32))
    k = W.f32_to_bf16_bits((raw((N, d)) + rng.normal(0, 2 ** 0.5, d)).astype(np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    return w, q, k, v


def test_attend_bf16_equals_textbook_on_dequantized_operands():
    w, q, k, v = _head(N=300, d=64)
    bq, bk = 32, 64
    qc, qs = quant.quantize_q(q, bq)
    kc, ks, mu = quant.quantize_k(k, bk)
    rows = np.arange(300)
    O = A.attend_bf16(qc, qs, kc, ks, v, rows, bq, bk, 0.125)
    Qd = qc.astype(np.float64) * np.repeat(qs, bq)[:300, None]
    Kd = kc.astype(np.float64) * np.repeat(ks, bk)[:300, None]
    Vf = W.bf16_bits_to_f32(v).astype(np.float64)
    np.testing.assert_allclose(O, _sdpa(Qd, Kd, Vf, 0.125), atol=1e-12)
    # and it approximates exact attention of the bf16 inputs closely
    ex = A.attention_fp64(W.bf16_bits_to_f32(q), W.bf16_bits_to_f32(k), Vf, 0.125)
    cos = (O * ex).sum() / np.linalg.norm(O) / np.linalg.norm(ex)
    assert cos > 0.9995 and np.abs(O - ex).max() < 2e-2


def test_quantized_pipeline_block_permutation_invariance():
    w, q, k, v = _head(N=256, d=64, seed=5)
    r1 = oracle.forward_head(q, k, v, np.arange(256), 64, 64, 0.125)
    order = [3, 1, 0, 2]
    perm = np.concatenate([np.arange(64) + 64 * o for o in order])
    r2 = oracle.forward_head(q, k[perm], v[perm], np.arange(256), 64, 64, 0.125)
    assert np.array_equal(r2["k_codes"], r1["k_codes"][perm])
    np.testing.assert_allclose(r2["out"], r1["out"], atol=1e-12)


def _online_loop(S, Vh, tile, round_p):
    """Online softmax written as its recurrence, one tile at a time:
    m <- max(m, max tile); acc, l rescaled by e^(m_old - m_new); P~ = e^(s - m);
    acc += round(448 P~)/448 * v; l += P~."""
    R, N = S.shape
    out = np.zeros((R, Vh.shape[1]))
    for r in range(R):
        m = -np.inf
        acc = np.zeros(Vh.shape[1])
        l = 0.0
        for t0 in range(0, N, tile):
            s = S[r, t0:t0 + tile]
            m_new = max(m, s.max())
            alpha = math.exp(m - m_new) if m != -np.inf else 0.0
            acc *= alpha
            l *= alpha
            p = np.exp(s - m_new)
            acc += (round_p(448.0 * p) / 448.0) @ Vh[t0:t0 + tile]
            l += p.sum()
            m = m_new
        out[r] = acc / l
    return out


def test_fp8_mirror_matches_stepwise_online_recurrence():
    w, q, k, v = _head(N=333, d=64, seed=6, dist="t3")
    qc, qs = quant.quantize_q(q, 64)
    kc, ks, mu = quant.quantize_k(k, 64)
    vc, vs = quant.quantize_v_fp8(v, 64)
    rows = np.array([0, 5, 100, 200, 332])
    O, E, hits = A.attend_fp8(qc, qs, kc, ks, vc, vs, rows, 64, 64, 0.125)
    S = A.logits(A.int_scores(qc[rows], kc), qs[rows // 64], np.repeat(ks, 64)[:333], 0.125)
    Vh = fp.e4m3_decode(vc) * np.repeat(vs, 64)[:333, None]
    ref = _online_loop(S, Vh, 64, lambda y: A.e4m3_round_f64(y)[0])
    np.testing.assert_allclose(O, ref, atol=1e-12)
    # tile width matters: a 128-key schedule rounds differently
    O128, _, _ = A.attend_fp8(qc, qs, kc, ks, vc, vs, rows, 64, 64, 0.125, kv_tile=128)
    np.testing.assert_allclose(O128, _online_loop(S, Vh, 128, lambda y: A.e4m3_round_f64(y)[0]), atol=1e-12)


def test_fp8_mirror_special_cases():
    w, q, k, v = _head(N=200, d=32, seed=7)
    qc, qs = quant.quantize_q(q, 64)
    kc, ks, mu = quant.quantize_k(k, 64)
    vc, vs = quant.quantize_v_fp8(v, 64)
    rows = np.arange(200)
    Vh = fp.e4m3_decode(vc) * np.repeat(vs, 64)[:200, None]
    # identity rounding: the mirror is the exact softmax over dequantized V
    O_id, _, _ = A.attend_fp8(qc, qs, kc, ks, vc, vs, rows, 64, 64, 0.2, round_p=lambda y: y)
    S = A.logits(A.int_scores(qc, kc), qs[rows // 64], np.repeat(ks, 64)[:200], 0.2)
    np.testing.assert_allclose(O_id, A.softmax_pv(S, Vh), atol=1e-12)
    # all logits equal (Q = 0): P~ = 1, 448 is exact in E4M3, output is the mean of V
    qz = np.zeros(200, np.int8)[:, None].repeat(32, 1)
    O0, E0, hits0 = A.attend_fp8(qz, np.zeros(4, np.float32), kc, ks, vc, vs, rows, 64, 64, 0.2)
    np.testing.assert_allclose(O0, np.repeat(Vh.mean(0, keepdims=True), 200, 0), atol=1e-12)
    assert hits0 == 0 and not E0.any()


def test_e4m3_round_f64_agrees_with_encoder_and_flags_midpoints():
    rng = np.random.default_rng(8)
    y = np.exp2(rng.uniform(-12, 8.8, 100_000))
    r, quantum, c = A.e4m3_round_f64(y)
    y32 = y.astype(np.float32)
    exact32 = y32.astype(np.float64) == y
    ref = fp.e4m3_decode(fp.e4m3_encode(y32))
    assert np.array_equal(r[exact32], ref[exact32])
    # a value exactly on a midpoint lands in the envelope
    w, q, k, v = _head(N=64, d=16, seed=9)
    qc, qs = quant.quantize_q(q, 64)
    kc, ks, mu = quant.quantize_k(k, 64)
    vc, vs = quant.quantize_v_fp8(v, 64)
    # two keys whose logit difference puts 448*P~ exactly halfway between 416 and 448
    qz = np.zeros((1, 16), np.int8)
    qz[0, 0] = 1
    kz = np.zeros((2, 16), np.int8)
    kz[0, 0] = 0
    kz[1, 0] = 1
    target = math.log(432.0 / 448.0)            # P~ of key 0 relative to key 1 (the max)
    O, E, hits = A.attend_fp8(qz, np.float32([1.0]), kz, np.float32([-target]), vc[:2], vs[:1],
                              np.array([0]), 64, 64, 1.0)
    assert hits >= 1 and E.max() > 0


def test_per_row_q_scales_help_heavy_tailed_q():
    """Finer Q scale groups bound each row's rounding by its own absmax: on
    heavy-tailed (Student-t) Q the per-row variant is much closer to the
    unquantized attention than 128-row blocks (a property of the
    quantization, checked against attention_fp64)."""
    import math
    w = W.get("wan14b-480p-fp8")
    q, k, v, _ = W.gen_head(w, 0, 0, N=2048)
    rows = np.arange(0, 2048, 8)
    f = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    exact = A.attention_fp64(f(q)[rows], f(k), f(v), w.scale)
    cos = {}
    for qb in (128, 1):
        qc, qs = quant.quantize_q(q, qb)
        kc, ks, _ = quant.quantize_k(k, 64)
        o = A.attend_bf16(qc, qs, kc, ks, v, rows, qb, 64, w.scale)
        cos[qb] = float((o * exact).sum() / math.sqrt((o * o).sum() * (exact * exact).sum()))
    assert cos[1] > cos[128] and 1 - cos[1] < 0.5 * (1 - cos[128]), cos
