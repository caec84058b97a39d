"""GPU parity of block-sparse attention (sqattn_forward_sparse /
sqattn_attend_quantized_sparse) against the oracle with the same mask, at the
dense path's bar: quantization bit-exact (shared with the dense step), the
output within max-abs 1e-2 (plus the FP8 envelope) and cosine >= 0.9999 over
the checked rows, rows of an empty mask row exactly 0.  With an all-ones mask
the sparse kernels must reproduce the dense kernels bit for bit.
"""
import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import MAX_ABS, MIN_COS, check_fp8, dev_bf16, host, out_metrics
import oracle

pytestmark = pytest.mark.gpu


def _masked_case(w, mask, N=None, d=None, B=None, H=None, pv=None, heads=None):
    pv = pv or w.pv
    q, k, v, rows = W.gen_inputs(w, N=N, d=d, B=B, H=H)
    B_, H_, N_, d_ = q.shape
    print(f"case sparse {w.name} B={B_} H={H_} N={N_} d={d_} pv={pv} density={mask.mean():.3f}", flush=True)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    M = torch.from_numpy(mask).cuda()
    out = sq.forward(Q, K, V, scale=w.scale, pv=pv, q_block=w.q_block, block_mask=M)
    torch.cuda.synchronize()
    out_h = host(out)
    idx = list(range(B_ * H_)) if heads is None else list(heads)
    g_rows, r_rows, e_rows = [], [], []
    hits = elements = 0
    for i in idx:
        b, h = divmod(i, H_)
        r = oracle.forward_head(q[b, h], k[b, h], v[b, h], rows[i], w.q_block, 64, w.scale, pv=pv,
                                block_mask=mask[b, h])
        g = out_h[b, h][rows[i]]
        empty = ~mask[b, h][rows[i] // 128].any(axis=1)
        assert not g[empty].any(), f"head {i}: rows of an empty mask row are not zero"
        g_rows.append(g)
        r_rows.append(r["out"])
        e_rows.append(r["envelope"])
        if pv == "fp8":
            hits += r["envelope_hits"]
            elements += len(rows[i]) * N_
    mt = out_metrics(g_rows, r_rows, e_rows if pv == "fp8" else None)
    print(f"  max_abs {mt['max_abs']:.3g} excess {mt['max_excess']:.3g} cos {mt['cos']:.7f}", flush=True)
    assert mt["max_excess"] <= MAX_ABS, mt
    assert mt["cos"] >= MIN_COS, mt
    if pv == "fp8":
        check_fp8(mt, hits, elements)
    return out


@pytest.mark.parametrize("pv", ["bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_sparse_small(pv, d):
    w = W.get(0)
    N, H = 1000, 3
    mask = W.gen_block_mask(1, H, N, 0.3, seed=11 + d)
    mask[0, 0, 1, :] = 0            # an empty query block
    mask[0, 1, 0, :2] = 0           # first tiles dropped for waves 0-3, kept for 4-7
    mask[0, 1, 1, :2] = 1
    mask[0, 2, :, -1] = 1           # the ragged last tile kept everywhere
    mask[0, 0, :, -1] = 0           # ... and dropped everywhere
    _masked_case(w, mask, N=N, d=d, B=1, H=H, pv=pv)


@pytest.mark.parametrize("pv", ["bf16", "fp8"])
def test_sparse_all_ones_equals_dense(pv):
    w = W.get(0)
    N, H, d = 777, 2, 128
    q, k, v, _ = W.gen_inputs(w, N=N, d=d, B=1, H=H)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    M = torch.ones((1, H, -(-N // 128), -(-N // 64)), dtype=torch.uint8, device="cuda")
    a = sq.forward(Q, K, V, scale=w.scale, pv=pv)
    b = sq.forward(Q, K, V, scale=w.scale, pv=pv, block_mask=M)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_sparse_empty_work_groups_and_zero_mask():
    w = W.get(0)
    N, H = 700, 2
    mask = np.zeros((1, H, -(-N // 128), -(-N // 64)), np.uint8)
    mask[0, 1, 4, 3] = 1            # a single kept block
    out = _masked_case(w, mask, N=N, d=64, B=1, H=H, pv="bf16")
    o = host(out)
    assert not o[0, 0].any() and not o[0, 1, :512].any() and np.abs(o[0, 1, 512:640]).max() > 0


def test_sparse_deterministic_and_kernel_entry():
    w = W.get(0)
    N, H, d = 900, 2, 128
    q, k, v, _ = W.gen_inputs(w, N=N, d=d, B=1, H=H)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    M = torch.from_numpy(W.gen_block_mask(1, H, N, 0.4, seed=5)).cuda()
    for pv in ("bf16", "fp8"):
        a = sq.forward(Q, K, V, scale=w.scale, pv=pv, block_mask=M)
        b = sq.forward(Q, K, V, scale=w.scale, pv=pv, block_mask=M)
        qi, qs, ki, ks, _ = sq.quantize_qk(Q, K)
        if pv == "fp8":
            vc, vs = sq.quantize_v_fp8(V)
            vr, vp = vc, sq.pack_v(vc, "fp8")
        else:
            vs, vr, vp = None, V, sq.pack_v(V, "bf16")
        c = sq.attend_packed(qi, qs, ki, ks, vp, vs, scale=w.scale, pv=pv, block_mask=M)
        e = sq.attend_quantized(qi, qs, ki, ks, vr, vs, scale=w.scale, pv=pv, block_mask=M)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(a, e), pv


@pytest.mark.parametrize("name,density", [("wan14b-480p", 0.15), ("wan14b-480p-fp8", 0.15)])
def test_sparse_full_size_sampled(name, density):
    """Full-size heads with a selector-like mask (local band + 15% random
    blocks), sampled rows of every 8th head against all keys."""
    w = W.get(name)
    mask = W.gen_block_mask(w.B, w.H, w.N, density, seed=w.index)
    _masked_case(w, mask, heads=range(0, w.B * w.H, 8))
