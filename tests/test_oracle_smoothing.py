"""Pins of the oracle's Q smoothing (quant.quantize_q_smoothed and the logit
bias of attention.smoothing_bias / smoothing_width).

Tied to: exact attention (with the quantization taken out, Q' K'^T plus the
bias is Q K'^T, so softmax equals unquantized float64 attention to 1e-12),
an invariance (adding a constant vector to every row of a block shifts the
mean by exactly that vector and leaves codes and scales unchanged), special
cases (a zero-mean block quantizes as plain Q, a block of equal rows too,
a huge offset is smoothed exactly), an exact emulation of the binary32 bias chain
the envelope term bounds, and the accuracy it buys on offset Q."""
import numpy as np

import workloads as W
from oracle import attention as A
from oracle import quant


def _f(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def _head(N=300, d=64, sigma=3.0, seed=11, idx=1):
    w = W.get(idx)
    q, k, v, _ = W.gen_inputs(w, N=N, d=d, B=1, H=1)
    q = W.add_channel_offset(q, sigma, seed)
    return w, q[0, 0], k[0, 0], v[0, 0]


def test_bias_restores_exact_attention_without_quantization():
    # Q' = fl32(Q - mu_b) as real values (no codes), K' likewise: the smoothed
    # logits Q' K'^T + mu_b K'^T are (Q' + mu_b) K'^T, whatever the block of
    # each row
    w, q, k, v = _head()
    N = q.shape[0]
    for qb in (64, 128):
        _, _, mu = quant.quantize_q_smoothed(q, qb)
        assert np.abs(mu).max() > 1.0                      # the offset is smoothed
        kc, ks, km = quant.quantize_k(k, 64)
        kp = quant.smooth_k(k, km).astype(np.float64)
        rows = np.arange(N)
        qp = np.concatenate([quant.smooth_k(q[b * qb:(b + 1) * qb], mu[b]) for b in range(-(-N // qb))])
        S = A.logits(qp.astype(np.float64) @ kp.T, np.ones(N), np.ones(N), w.scale)
        S = S + A.smoothing_bias(mu, kp, rows, qb) * w.scale
        O = A.softmax_pv(S, _f(v))
        # Q' + mu_b in float64 is Q up to the binary32 rounding of Q'
        qrec = qp.astype(np.float64) + mu.astype(np.float64)[rows // qb]
        assert np.abs(qrec - _f(q)).max() <= 2.0 ** -23 * np.abs(qp).max()
        ref = A.attention_fp64(qrec, kp, _f(v), w.scale)
        assert np.abs(O - ref).max() <= 1e-12 * np.abs(ref).max()


def test_constant_shift_of_a_block():
    # values on a 1/8 grid within +-16: q + c stays exact in bf16 and the
    # block mean moves by exactly c; Q' and hence codes and scales do not move
    rng = np.random.default_rng(3)
    x = rng.integers(-64, 64, size=(256, 64)) / 8.0
    c = rng.integers(-16, 16, size=64) / 8.0
    q0 = W.f32_to_bf16_bits(x.astype(np.float32))
    q1 = W.f32_to_bf16_bits((x + c).astype(np.float32))
    assert np.array_equal(_f(q1), x + c)
    c0, s0, m0 = quant.quantize_q_smoothed(q0, 128)
    c1, s1, m1 = quant.quantize_q_smoothed(q1, 128)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert np.array_equal(m1.astype(np.float64), m0.astype(np.float64) + c[None, :])


def test_zero_mean_block_is_plain_quantization():
    rng = np.random.default_rng(4)
    half = rng.standard_normal((64, 32))
    x = np.concatenate([half, -half])                    # every channel sums to exactly 0
    qb = W.f32_to_bf16_bits(x.astype(np.float32))
    qb = np.concatenate([qb, qb ^ np.uint16(0x8000)])[:128]   # rows and their negations
    c, s, mu = quant.quantize_q_smoothed(qb, 128)
    cp, sp = quant.quantize_q(qb, 128)
    assert not mu.any() and np.array_equal(c, cp) and np.array_equal(s, sp)


def test_constant_block_is_plain_and_any_offset_is_smoothed():
    # a block whose rows are all equal has Q' = 0 and s = 0: quantized
    # plainly; a huge offset (|mu| = 2^14 against Q' of +-128) is smoothed
    x = np.tile(np.linspace(-3, 3, 64), (64, 1))
    qb = W.f32_to_bf16_bits(x.astype(np.float32))
    c, s, mu = quant.quantize_q_smoothed(qb, 64)
    assert not mu.any() and np.array_equal(c, quant.quantize_q(qb, 64)[0])
    x = np.where(np.arange(64)[None, :] % 2 == np.arange(64)[:, None] % 2, 128.0, -128.0) + 16384.0 * (
        np.arange(64) % 3 - 1)[None, :]
    qb = W.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(qb), x)
    c, s, mu = quant.quantize_q_smoothed(qb, 64)
    assert np.array_equal(mu[0], (16384.0 * (np.arange(64) % 3 - 1)).astype(np.float32))
    assert s[0] == np.float32(128.0) / np.float32(127.0) and np.array_equal(np.abs(c), np.full((64, 64), 127))


def _fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _kernel_bias(mu, kp, sq, sk):
    """The bias as the module notes describe the FP8 kernel computing it: 16
    FMA chains of 8 terms (channel order), summed pairwise in binary32,
    divided by fl32(sQ sK) (correctly rounded); binary32."""
    f32 = np.float32
    d = mu.shape[-1]
    part = np.zeros(mu.shape[:-1] + (kp.shape[0], d // 8), f32)
    for g in range(d // 8):
        acc = np.zeros(mu.shape[:-1] + (kp.shape[0],), f32)
        for c in range(8 * g, 8 * g + 8):
            acc = _fma32(np.broadcast_to(mu[..., None, c], acc.shape), np.broadcast_to(kp[:, c], acc.shape), acc)
        part[..., g] = acc
    while part.shape[-1] > 1:
        part = (part[..., 0::2] + part[..., 1::2]).astype(f32)
    den = (sq.astype(f32)[:, None] * sk.astype(f32)[None, :]).astype(f32)
    q = (part[..., 0].astype(np.float64) / np.where(den == 0, 1, den)).astype(f32)
    return np.where(den == 0, f32(0), q)


def test_biased_scores_within_smoothing_width():
    # fl32(S + bias) with the binary32 bias deviates from the exact biased
    # logit by no more than the per-row width smoothing_width charges for it
    w, q, k, v = _head(N=512, d=128, sigma=4.0, idx=3)
    qb = 128
    qc, qs, mu = quant.quantize_q_smoothed(q, qb)
    kc, ks, km = quant.quantize_k(k, 64)
    kp = quant.smooth_k(k, km)
    rows = np.arange(0, 512, 3)
    D = A.int_scores(qc[rows], kc)                                                  # exact integers
    sk = np.repeat(ks, 64)[:512]
    sq = qs[rows // qb]
    unit = sq[:, None].astype(np.float64) * sk[None, :]                             # sQ sK
    exact = D + A.smoothing_bias(mu, kp, rows, qb) / unit                           # in units of sQ sK
    beta = _kernel_bias(mu[rows // qb], kp, sq, sk)
    v = (D.astype(np.float32) + beta).astype(np.float32).astype(np.float64)         # fl32(S + bias)
    c = unit * w.scale * np.log2(np.e)
    M = np.abs(exact * c).max(axis=1, keepdims=True)
    rel = np.log(2.0) * (c * np.abs(v - exact)).max(axis=1, keepdims=True)
    width = A.smoothing_width(mu, kp, rows, qb, w.scale, M)
    assert np.all(rel <= width), float((rel / width).max())
    assert (rel / width).max() > 1.0 / 64                   # not loose by orders of magnitude


def test_smoothing_reduces_error_on_offset_q():
    # Q with per-channel offsets of sigma 4: per-block smoothing brings the
    # bf16-path output closer to unquantized attention than plain per-block
    # scales, and at least as close as one scale per row
    w, q, k, v = _head(N=1024, d=128, sigma=4.0, idx=2)
    kc, ks, km = quant.quantize_k(k, 64)
    kp = quant.smooth_k(k, km)
    rows = np.arange(0, 1024, 4)
    ref = A.attention_fp64(_f(q)[rows], _f(k), _f(v), w.scale)
    err = {}
    qc, qs = quant.quantize_q(q, 128)
    err["plain"] = A.attend_bf16(qc, qs, kc, ks, v, rows, 128, 64, w.scale)
    qc, qs = quant.quantize_q(q, 1)
    err["per_row"] = A.attend_bf16(qc, qs, kc, ks, v, rows, 1, 64, w.scale)
    qc, qs, mu = quant.quantize_q_smoothed(q, 128)
    err["smoothed"] = A.attend_bf16(qc, qs, kc, ks, v, rows, 128, 64, w.scale, q_mean=mu, k_smooth=kp)
    e = {n: float(np.abs(o - ref).mean()) for n, o in err.items()}
    assert e["smoothed"] < 0.7 * e["plain"] and e["smoothed"] <= e["per_row"], e
