"""GPU: attention with the per-token q/k RMSNorm fused into the quantization
(sqattn_forward_qknorm) against the same attention on Q and K normalized by
the oracle (oracle.norm.qk_rmsnorm: exact mean square, binary32 factor and
weight, nearest-even bf16) and handed to the plain forward.

The two runs share every kernel after the normalization, so their outputs
must be equal bit for bit: any difference in the normalized values, their
bf16 rounding or the layout handling shows up.  Q, K and V are views of a
fused QKV projection output [B, N, 3, H, d] (the layout the entry point is
for); the plain forward gets contiguous normalized tensors.
"""
import math

import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import MAX_ABS, MIN_COS, dev_bf16, host
from oracle import attention, norm, quant

pytestmark = pytest.mark.gpu


def _qkv(B, N, H, d, seed, kind="normal"):
    """bf16 [B, N, 3, H, d]: q and k with per-token magnitudes spread over
    2^-8 .. 2^8 (the normalization undoes them), a K channel offset, V standard
    normal, and for kind "edge" a zero token, a huge token, a tiny one and one
    with a single non-zero value in q and k."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, 3, H, d))
    x[:, :, :2] *= np.ldexp(1.0, rng.integers(-8, 9, (B, N, 1, 1, 1)))
    x[:, :, 1] += rng.standard_normal(d) * 1.4
    if kind == "edge":
        x[0, 0, :2] = 0.0
        x[0, 1, :2] *= 2.0 ** 100
        x[0, 2, :2] *= 2.0 ** -100
        x[-1, -1, :2] = 0.0
        x[-1, -1, :2, 0, 0] = 3.0
    bits = W.f32_to_bf16_bits(x.astype(np.float32))
    return bits, dev_bf16(bits)


def _gamma(H, d, seed, kind):
    if kind is None:
        return None
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal(H * d) * 0.3 + 1.0).astype(np.float32)
    if kind == "signs":
        g[::7] = 0.0
        g[1::5] *= -1.0
    return g


def _views(qkv):
    return [qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)]   # [B, H, N, d], head stride d


@pytest.mark.parametrize("pv,d,gk,q_block,out_dtype,sparse", [
    ("bf16", 128, "plain", 128, torch.float32, False),
    ("bf16", 64, None, 128, torch.bfloat16, False),
    ("fp8", 128, "signs", 128, torch.float32, False),
    ("fp8", 64, "plain", 1, torch.float32, False),
    ("bf16", 128, "plain", 1, torch.bfloat16, True),
])
def test_fused_equals_normalize_then_attend(pv, d, gk, q_block, out_dtype, sparse):
    B, N, H = 2, 700, 3
    eps = 1e-6
    print(f"case qknorm pv={pv} d={d} gamma={gk} q_block={q_block} out={out_dtype} sparse={sparse}", flush=True)
    bits, qkv = _qkv(B, N, H, d, seed=d + (3 if pv == "fp8" else 0), kind="edge")
    gq, gkk = _gamma(H, d, 1, gk), _gamma(H, d, 2, gk)
    q, k, v = _views(qkv)
    mask = W.gen_block_mask(B, H, N, 0.3, seed=5) if sparse else None
    m = torch.from_numpy(mask).cuda() if sparse else None
    G = lambda g: None if g is None else torch.from_numpy(g).cuda()
    fused = sq.forward_qknorm(q, k, v, G(gq), G(gkk), eps, pv=pv, q_block=q_block, out_dtype=out_dtype,
                              block_mask=m)
    # the oracle's normalization, then the plain forward on contiguous tensors
    qb = np.ascontiguousarray(bits[:, :, 0].transpose(0, 2, 1, 3))
    kb = np.ascontiguousarray(bits[:, :, 1].transpose(0, 2, 1, 3))
    qn, kn = norm.qk_rmsnorm(qb, gq, eps), norm.qk_rmsnorm(kb, gkk, eps)
    plain = sq.forward(dev_bf16(qn), dev_bf16(kn), v.contiguous(), pv=pv, q_block=q_block, out_dtype=out_dtype,
                       block_mask=m)
    torch.cuda.synchronize()
    a, b = host(fused.float()), host(plain.float())
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"max diff {np.nanmax(np.abs(a - b))}"


def test_against_the_oracle():
    """A small case end to end against the oracle's attention on the
    normalized tensors: output within the parity tolerance."""
    B, N, H, d = 1, 300, 2, 64
    eps = 1e-6
    bits, qkv = _qkv(B, N, H, d, seed=11)
    gq, gkk = _gamma(H, d, 3, "plain"), _gamma(H, d, 4, "plain")
    q, k, v = _views(qkv)
    out = sq.forward_qknorm(q, k, v, torch.from_numpy(gq).cuda(), torch.from_numpy(gkk).cuda(), eps, q_block=64)
    torch.cuda.synchronize()
    o = host(out)
    qn = norm.qk_rmsnorm(np.ascontiguousarray(bits[:, :, 0].transpose(0, 2, 1, 3)), gq, eps)
    kn = norm.qk_rmsnorm(np.ascontiguousarray(bits[:, :, 1].transpose(0, 2, 1, 3)), gkk, eps)
    vb = np.ascontiguousarray(bits[:, :, 2].transpose(0, 2, 1, 3))
    rows = np.arange(N)
    for h in range(H):
        qc, qs = quant.quantize_q(qn[0, h], 64)
        kc, ks, _ = quant.quantize_k(kn[0, h], 64)
        ref = attention.attend_bf16(qc, qs, kc, ks, vb[0, h], rows, 64, 64, 1.0 / math.sqrt(d))
        got = o[0, h].astype(np.float64)
        err = np.abs(got - ref).max()
        cos = float((got * ref).sum() / (np.linalg.norm(got) * np.linalg.norm(ref)))
        print(f"  head {h}: max abs {err:.3g} cos {cos:.8f}", flush=True)
        assert err <= MAX_ABS and cos >= MIN_COS


def test_wan_shape_tokens():
    """Wan-1.3B-shaped heads (H = 12, d = 128, H*d = 1536 features per token)
    over 4096 tokens: fused equals normalize-then-attend."""
    B, N, H, d = 1, 4096, 12, 128
    eps = 1e-6
    print(f"case qknorm B={B} N={N} H={H} d={d}", flush=True)
    bits, qkv = _qkv(B, N, H, d, seed=21)
    gq, gkk = _gamma(H, d, 5, "plain"), _gamma(H, d, 6, "plain")
    q, k, v = _views(qkv)
    fused = sq.forward_qknorm(q, k, v, torch.from_numpy(gq).cuda(), torch.from_numpy(gkk).cuda(), eps)
    qn = norm.qk_rmsnorm(np.ascontiguousarray(bits[:, :, 0].transpose(0, 2, 1, 3)), gq, eps)
    kn = norm.qk_rmsnorm(np.ascontiguousarray(bits[:, :, 1].transpose(0, 2, 1, 3)), gkk, eps)
    plain = sq.forward(dev_bf16(qn), dev_bf16(kn), v.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)


def test_rejects_head_major_layout():
    B, N, H, d = 1, 128, 2, 64
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sq.SqattnError, match="contiguous"):
        sq.forward_qknorm(q, q, q, None, None, 1e-6)
