"""GPU parity of Q smoothing (opts.smooth_q) against the oracle
(quant.quantize_q_smoothed and the logit bias of attention.smoothing_bias).

Inputs: the workloads' seeded Q/K/V with a per-channel Q offset added
(workloads.add_channel_offset), the outliers smoothing targets; on the FP8
path the oracle's envelope includes the width the kernel's rounded integer
bias takes (attention.smoothing_width)."""
import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import MAX_ABS, MIN_COS, check_fp8, dev_bf16, host, oracle_heads, out_metrics
from oracle import attention as A

pytestmark = pytest.mark.gpu

# the smoothing term widens the FP8 ambiguity band by up to ln 2 (0.5 + ...)
# units of c: the fraction of flagged P elements may grow to a few 1e-3
SMOOTH_ENV_HIT_FRAC = 5e-3


def _case(idx, N, d, B, H, q_block, sigma=4.0, rows_all=True, heads=None, tol=MAX_ABS):
    w = W.get(idx)
    q, k, v, rows = W.gen_inputs(w, N=N, d=d, B=B, H=H)
    q = W.add_channel_offset(q, sigma, seed=idx * 1000 + N)
    if rows_all:
        rows = [np.arange(N)] * (B * H)
    print(f"case {w.name} B={B} H={H} N={N} d={d} q_block={q_block} pv={w.pv} smooth sigma={sigma}", flush=True)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out = sq.forward(Q, K, V, scale=w.scale, pv=w.pv, q_block=q_block, smooth_q=True)
    torch.cuda.synchronize()
    ref = oracle_heads(q, k, v, rows, q_block, w.scale, w.pv, heads=heads, smooth_q=True)
    idxs = [i for i in range(B * H) if ref[i] is not None]
    if N > 1:  # one row per block leaves Q' = 0 (s = 0): quantized plainly
        assert any(ref[i]["q_mean"].any() for i in idxs), "no block was smoothed"
    out_h = host(out)
    g_rows, r_rows, e_rows = [], [], []
    for i in idxs:
        b, h = divmod(i, H)
        g_rows.append(out_h[b, h][rows[i]])
        r_rows.append(ref[i]["out"])
        e_rows.append(ref[i]["envelope"])
    m = out_metrics(g_rows, r_rows, e_rows if w.pv == "fp8" else None)
    print(f"  max_abs={m['max_abs']:.3e} excess={m['max_excess']:.3e} cos={m['cos']:.8f}", flush=True)
    assert np.isfinite(out_h).all()
    assert m["max_excess"] <= tol and m["cos"] >= MIN_COS, m
    if w.pv == "fp8":
        hits = sum(ref[i]["envelope_hits"] for i in idxs)
        elems = sum(len(rows[i]) * N for i in idxs)
        check_fp8(m, hits, elems, bound_hits=False)
        assert hits / elems <= SMOOTH_ENV_HIT_FRAC, (hits, elems)
    return w, q, k, v, out_h, rows


@pytest.mark.parametrize("q_block", [64, 128, 256])
def test_bf16_wan13b_shape(q_block):
    _case(1, N=700, d=128, B=1, H=3, q_block=q_block)


@pytest.mark.parametrize("q_block", [64, 128, 256])
def test_fp8_wan14b_shape(q_block):
    _case(3, N=700, d=128, B=1, H=2, q_block=q_block)


@pytest.mark.parametrize("N", [1, 63, 65, 300, 513])
@pytest.mark.parametrize("pv_idx", [1, 3])
def test_ragged_and_d64(N, pv_idx):
    # work-groups whose later waves lie past N, partial last blocks, d = 64
    _case(pv_idx, N=N, d=64, B=2, H=1, q_block=128)


def test_no_offset_and_large_offset():
    # without an offset every block is smoothed with a small mean; a large
    # offset puts most of each logit into the bias.  Its softmax is peaked
    # (the largest P of a row ~0.7): the bf16 path's rounding of P (2^-9
    # relative, not mirrored by the oracle) alone then moves an output by up
    # to 2^-9 (|V_j| + |O|) <= 2^-8 max|V| (an emulation of that rounding
    # gives 0.0131 on these rows), so its bar is 2^-8 max|V|; the FP8 path
    # mirrors its rounding and keeps the default bar
    _case(1, N=400, d=128, B=1, H=2, q_block=128, sigma=0.0)
    w = W.get(1)
    v = W.gen_inputs(w, N=400, d=128, B=1, H=2)[2]
    _case(1, N=400, d=128, B=1, H=2, q_block=128, sigma=20.0,
          tol=2.0 ** -8 * float(np.abs(W.bf16_bits_to_f32(v)).max()))
    _case(3, N=400, d=128, B=1, H=2, q_block=128, sigma=20.0)


@pytest.mark.parametrize("idx", [1, 3])
def test_full_size_sampled(idx):
    # the Wan-1.3B (bf16) and Wan-14B (fp8) shapes at full N, two heads
    # checked on the workload's sampled rows
    w = W.get(idx)
    _case(idx, N=w.N, d=w.d, B=w.B, H=w.H, q_block=w.q_block, rows_all=False, heads=[0, w.H - 1])


def test_smoothing_reduces_error_on_offset_q():
    # the accuracy the option buys: against unquantized float64 attention on
    # the same bf16 inputs, smoothed per-block Q beats plain per-block Q
    w = W.get(1)
    q, k, v, _ = W.gen_inputs(w, N=2048, d=128, B=1, H=2)
    q = W.add_channel_offset(q, 4.0, seed=5)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o_s = host(sq.forward(Q, K, V, scale=w.scale, q_block=128, smooth_q=True))
    o_p = host(sq.forward(Q, K, V, scale=w.scale, q_block=128))
    f = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    rows = np.arange(0, 2048, 8)
    e_s = e_p = 0.0
    for h in range(2):
        ref = A.attention_fp64(f(q[0, h])[rows], f(k[0, h]), f(v[0, h]), w.scale)
        e_s += np.abs(o_s[0, h][rows] - ref).mean()
        e_p += np.abs(o_p[0, h][rows] - ref).mean()
    print(f"  mean abs error vs fp64: smoothed {e_s / 2:.3e}, plain {e_p / 2:.3e}", flush=True)
    assert e_s < 0.6 * e_p


def test_smoothing_refused_where_unsupported():
    w = W.get(1)
    q, k, v, _ = W.gen_inputs(w, N=128, d=64, B=1, H=1)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    with pytest.raises(RuntimeError, match="Q smoothing"):
        sq.forward(Q, K, V, q_block=1, smooth_q=True)
    m = torch.ones((1, 1, 1, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="dense"):
        sq.forward(Q, K, V, smooth_q=True, block_mask=m)
