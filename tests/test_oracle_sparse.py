"""Pins of the oracle's block-sparse attention (a block mask over 128-row query
blocks x 64-key tiles; oracle/attention.py, block_mask arguments).

What ties it to something other than itself:
  * an all-ones mask is the dense oracle, bit for bit;
  * for the rows of one query block, the masked result equals the dense
    oracle run on the kept tiles alone (keys, scales and V compacted): a
    different route that never forms a -inf logit;
  * brute force on a tiny head: per row, Python floats over the kept keys;
  * K codes and (finite) V rows of dropped tiles do not reach the dropped
    rows' output;
  * a query block with no kept tile yields zeros.
"""
import math

import numpy as np

from oracle import attention, quant
import workloads as W


def _head(N, d=64, seed=0):
    w = W.get("tiny-256x64")
    q, k, v, _ = W.gen_head(w, 0, 0, N=N, d=d) if seed == 0 else _rand(N, d, seed)
    qc, qs = quant.quantize_q(q, 128)
    kc, ks, _ = quant.quantize_k(k, 64)
    vc, vs = quant.quantize_v_fp8(v, 64)
    return dict(q=q, k=k, v=v, qc=qc, qs=qs, kc=kc, ks=ks, vc=vc, vs=vs, N=N, scale=1.0 / math.sqrt(d))


def _rand(N, d, seed):
    rng = np.random.default_rng(seed)
    f = lambda a: W.f32_to_bf16_bits(a.astype(np.float32))
    return f(rng.standard_normal((N, d))), f(rng.standard_normal((N, d)) + 1.0), f(rng.standard_normal((N, d))), None


def _mask(N, rng, p=0.5):
    m = (rng.random((-(-N // 128), -(-N // 64))) < p).astype(np.uint8)
    return m


def test_all_ones_mask_is_dense():
    h = _head(300)
    N = h["N"]
    rows = np.arange(N)
    ones = np.ones((3, 5), np.uint8)
    a = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"])
    b = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"], block_mask=ones)
    np.testing.assert_array_equal(a, b)
    o1, e1, _ = attention.attend_fp8(h["qc"], h["qs"], h["kc"], h["ks"], h["vc"], h["vs"], rows, 128, 64, h["scale"])
    o2, e2, _ = attention.attend_fp8(h["qc"], h["qs"], h["kc"], h["ks"], h["vc"], h["vs"], rows, 128, 64, h["scale"],
                                     block_mask=ones)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(e1, e2)


def test_masked_rows_equal_dense_on_kept_tiles():
    h = _head(520, seed=3)
    N = h["N"]
    rng = np.random.default_rng(4)
    m = _mask(N, rng)
    m[:, -1] = 1  # keep the ragged last tile in some rows
    m[1, -1] = 0
    for qb in range(m.shape[0]):
        T = np.nonzero(m[qb])[0]
        rows = np.arange(128 * qb, min(N, 128 * qb + 128))
        if T.size == 0:
            continue
        keys = np.concatenate([np.arange(64 * t, min(N, 64 * t + 64)) for t in T])
        got = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"],
                                    block_mask=m)
        ref = attention.attend_bf16(h["qc"], h["qs"], h["kc"][keys], h["ks"][T], h["v"][keys], rows, 128, 64,
                                    h["scale"])
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
        go, ge, _ = attention.attend_fp8(h["qc"], h["qs"], h["kc"], h["ks"], h["vc"], h["vs"], rows, 128, 64,
                                         h["scale"], block_mask=m)
        ro, re, _ = attention.attend_fp8(h["qc"], h["qs"], h["kc"][keys], h["ks"][T], h["vc"][keys], h["vs"][T],
                                         rows, 128, 64, h["scale"])
        np.testing.assert_allclose(go, ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ge, re, rtol=1e-9, atol=1e-15)


def test_brute_force_tiny():
    h = _head(200, seed=5)
    N = h["N"]
    m = np.array([[1, 0, 1, 0], [0, 1, 0, 1]], np.uint8)
    rows = np.array([0, 7, 127, 128, 150, 199])
    got = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"], block_mask=m)
    V = W.bf16_bits_to_f32(h["v"]).astype(np.float64)
    for i, r in enumerate(rows):
        kept = [j for j in range(N) if m[r // 128, j // 64]]
        s = []
        for j in kept:
            dot = sum(int(a) * int(b) for a, b in zip(h["qc"][r], h["kc"][j]))
            s.append(dot * float(h["qs"][r // 128]) * float(h["ks"][j // 64]) * h["scale"])
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        want = [sum(e[t] * V[j, c] for t, j in enumerate(kept)) / tot for c in range(V.shape[1])]
        np.testing.assert_allclose(got[i], want, rtol=1e-11, atol=1e-12)


def test_dropped_tiles_do_not_reach_output():
    h = _head(384, seed=6)
    N = h["N"]
    m = np.array([[1, 1, 0, 0, 1, 0], [0, 1, 1, 1, 0, 0], [1, 0, 0, 0, 0, 1]], np.uint8)
    rows = np.arange(N)
    base = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"], block_mask=m)
    bo, _, _ = attention.attend_fp8(h["qc"], h["qs"], h["kc"], h["ks"], h["vc"], h["vs"], rows, 128, 64, h["scale"],
                                    block_mask=m)
    rng = np.random.default_rng(7)
    for qb in range(3):
        kc, v, vc = h["kc"].copy(), h["v"].copy(), h["vc"].copy()
        for t in np.nonzero(m[qb] == 0)[0]:
            sl = slice(64 * t, 64 * t + 64)
            kc[sl] = rng.integers(-127, 128, kc[sl].shape)
            v[sl] = W.f32_to_bf16_bits((rng.standard_normal(v[sl].shape) * 1e3).astype(np.float32))
            vc[sl] = rng.integers(0, 0x7E, vc[sl].shape).astype(np.uint8)
        r = np.arange(128 * qb, 128 * qb + 128)
        got = attention.attend_bf16(h["qc"], h["qs"], kc, h["ks"], v, r, 128, 64, h["scale"], block_mask=m)
        np.testing.assert_array_equal(got, base[r])
        go, _, _ = attention.attend_fp8(h["qc"], h["qs"], kc, h["ks"], vc, h["vs"], r, 128, 64, h["scale"],
                                        block_mask=m)
        np.testing.assert_array_equal(go, bo[r])


def test_empty_query_block_is_zero():
    h = _head(256, seed=8)
    m = np.array([[0, 0, 0, 0], [1, 0, 0, 1]], np.uint8)
    rows = np.arange(256)
    o = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"], block_mask=m)
    assert not o[:128].any() and np.abs(o[128:]).max() > 0
    f, e, _ = attention.attend_fp8(h["qc"], h["qs"], h["kc"], h["ks"], h["vc"], h["vs"], rows, 128, 64, h["scale"],
                                   block_mask=m)
    assert not f[:128].any() and not e[:128].any() and np.abs(f[128:]).max() > 0
    z = attention.attend_bf16(h["qc"], h["qs"], h["kc"], h["ks"], h["v"], rows, 128, 64, h["scale"],
                              block_mask=np.zeros((2, 4), np.uint8))
    assert not z.any()
