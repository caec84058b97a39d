"""GPU: strided operands (sqattn_forward_strided) and the composition of a
DiT attention block without layout copies.

Q, K, V taken as views of a fused QKV projection output [B, N, 3, H, d] and
the output written into a [B, N, H, d] tensor must give exactly the bytes of
the contiguous entry points on the same values (the kernels are the same;
only addresses differ).  The block test chains the W8A8 QKV projection,
attention on its output in place, and the W8A8 output projection on the
attention output in place, against the same chain with explicit copies.
"""
import math

import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _qkv(B, N, H, d, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    qkv = torch.randn((B, N, 3, H, d), generator=g, device="cuda").to(torch.bfloat16)
    qkv[:, :, 1] += torch.randn((d,), generator=g, device="cuda").to(torch.bfloat16) * 1.4
    return qkv


@pytest.mark.parametrize("pv,d,out_dtype,sparse", [
    ("bf16", 128, torch.float32, False),
    ("bf16", 64, torch.bfloat16, False),
    ("fp8", 128, torch.bfloat16, False),
    ("fp8", 64, torch.float32, True),
    ("bf16", 128, torch.bfloat16, True),
])
def test_strided_views_equal_contiguous(pv, d, out_dtype, sparse):
    B, N, H = 2, 700, 3
    print(f"case strided pv={pv} d={d} out={out_dtype} sparse={sparse}", flush=True)
    qkv = _qkv(B, N, H, d, seed=d + (1 if sparse else 0))
    q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))   # [B,H,N,d] views
    assert not q.is_contiguous()
    mask = torch.from_numpy(W.gen_block_mask(B, H, N, 0.3, seed=3)).cuda() if sparse else None
    ob = torch.empty((B, N, H, d), dtype=out_dtype, device="cuda")
    o_view = ob.permute(0, 2, 1, 3)
    sq.forward(q, k, v, pv=pv, out=o_view, block_mask=mask)
    ref = sq.forward(q.contiguous(), k.contiguous(), v.contiguous(), pv=pv, out_dtype=out_dtype, block_mask=mask)
    torch.cuda.synchronize()
    assert torch.equal(o_view, ref)


def test_strided_validation():
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    bad = torch.zeros((1, 2, 64, 72), dtype=torch.bfloat16, device="cuda")[..., :64]   # rows 16-byte aligned
    out = sq.forward(bad, q, q)   # strides (9216, 4608, 72): multiples of 8
    torch.cuda.synchronize()
    odd = torch.zeros((1, 2, 64, 68), dtype=torch.bfloat16, device="cuda")[..., :64]   # row stride 68
    with pytest.raises(sq.SqattnError):
        sq.forward(odd, q, q)


def test_dit_attention_block_without_copies():
    """x -> W8A8 QKV projection -> attention on its output in place ->
    W8A8 output projection on the attention output in place, against the
    same chain with explicit layout copies (bit for bit)."""
    B, N, H, d = 1, 1000, 4, 128
    C = H * d
    rng = np.random.default_rng(0)
    x = dev_bf16(W.f32_to_bf16_bits(rng.standard_normal((B * N, C)).astype(np.float32)))
    wqkv = dev_bf16(W.f32_to_bf16_bits((rng.standard_normal((3 * C, C)) / math.sqrt(C)).astype(np.float32)))
    wo = dev_bf16(W.f32_to_bf16_bits((rng.standard_normal((C, C)) / math.sqrt(C)).astype(np.float32)))
    bqkv = torch.from_numpy(rng.standard_normal(3 * C).astype(np.float32)).cuda()
    bo = torch.from_numpy(rng.standard_normal(C).astype(np.float32)).cuda()
    wqc, wqs = sq.w8a8_quantize(wqkv)
    woc, wos = sq.w8a8_quantize(wo)
    for pv in ("bf16", "fp8"):
        print(f"case dit block pv={pv} N={N} H={H} d={d}", flush=True)
        y = sq.w8a8_linear(x, wqc, wqs, bias=bqkv, out_dtype=torch.bfloat16)          # [B*N, 3C]
        qkv = y.view(B, N, 3, H, d)
        a = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
        sq.forward(*(qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)), pv=pv, out=a.permute(0, 2, 1, 3))
        z = sq.w8a8_linear(a.view(B * N, C), woc, wos, bias=bo, out_dtype=torch.bfloat16)
        # the same chain with copies into the contiguous layouts
        qc, kc, vc = (qkv[:, :, i].permute(0, 2, 1, 3).contiguous() for i in range(3))
        a2 = sq.forward(qc, kc, vc, pv=pv, out_dtype=torch.bfloat16)                    # [B,H,N,d]
        z2 = sq.w8a8_linear(a2.permute(0, 2, 1, 3).contiguous().view(B * N, C), woc, wos, bias=bo,
                            out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(a.permute(0, 2, 1, 3), a2)
        assert torch.equal(z, z2)
        assert torch.isfinite(z.float()).all()


def test_dit_block_with_fused_norms():
    """A Wan-style DiT attention block from the library's fused pieces, with
    no normalized tensor and no layout copy in memory:
      LayerNorm (modulation as gamma = 1 + scale, beta = shift) fused into the
      W8A8 QKV projection -> attention with the q/k RMSNorm fused, on views of
      the projection output -> W8A8 output projection on the attention output
      in place;
    against the chain taken step by step: LayerNorm + quantization, GEMM, the
    q/k normalization by the oracle into contiguous bf16 tensors, the plain
    forward, a copy into the projection layout, the output projection.  Bit
    for bit."""
    from oracle import norm
    B, N, H, d = 1, 900, 4, 128
    C = H * d
    rng = np.random.default_rng(1)
    xb = W.f32_to_bf16_bits((rng.standard_normal((B * N, C)) * 3 + 0.5).astype(np.float32))
    x = dev_bf16(xb)
    f = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()
    gamma, beta = f(1 + 0.2 * rng.standard_normal(C)), f(0.1 * rng.standard_normal(C))
    gq, gk = (1 + 0.1 * rng.standard_normal(C)).astype(np.float32), (1 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    wqkv = dev_bf16(W.f32_to_bf16_bits((rng.standard_normal((3 * C, C)) / math.sqrt(C)).astype(np.float32)))
    wo = dev_bf16(W.f32_to_bf16_bits((rng.standard_normal((C, C)) / math.sqrt(C)).astype(np.float32)))
    bqkv, bo = f(rng.standard_normal(3 * C)), f(rng.standard_normal(C))
    wqc, wqs = sq.w8a8_quantize(wqkv)
    woc, wos = sq.w8a8_quantize(wo)
    for pv in ("bf16", "fp8"):
        print(f"case dit block fused norms pv={pv} N={N} H={H} d={d}", flush=True)
        y = sq.w8a8_linear_layernorm(x, wqc, wqs, gamma=gamma, beta=beta, eps=1e-6, bias=bqkv,
                                     out_dtype=torch.bfloat16)                          # [B*N, 3C]
        qkv = y.view(B, N, 3, H, d)
        a = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
        sq.forward_qknorm(*(qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)), torch.from_numpy(gq).cuda(),
                          torch.from_numpy(gk).cuda(), 1e-6, pv=pv, out=a.permute(0, 2, 1, 3))
        z = sq.w8a8_linear(a.view(B * N, C), woc, wos, bias=bo, out_dtype=torch.bfloat16)
        # step by step
        xc, xs, _, _ = sq.w8a8_layernorm_quantize(x, gamma, beta, 1e-6)
        y2 = sq.w8a8_gemm(xc, xs, wqc, wqs, bias=bqkv, out_dtype=torch.bfloat16)
        yh = y2.view(B, N, 3, H, d).cpu().view(torch.int16).numpy().view(np.uint16)
        qn = norm.qk_rmsnorm(np.ascontiguousarray(yh[:, :, 0].transpose(0, 2, 1, 3)), gq, 1e-6)
        kn = norm.qk_rmsnorm(np.ascontiguousarray(yh[:, :, 1].transpose(0, 2, 1, 3)), gk, 1e-6)
        vc = y2.view(B, N, 3, H, d)[:, :, 2].permute(0, 2, 1, 3).contiguous()
        a2 = sq.forward(dev_bf16(qn), dev_bf16(kn), vc, pv=pv, out_dtype=torch.bfloat16)   # [B,H,N,d]
        z2 = sq.w8a8_linear(a2.permute(0, 2, 1, 3).contiguous().view(B * N, C), woc, wos, bias=bo,
                            out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        assert torch.equal(a.permute(0, 2, 1, 3), a2)
        assert torch.equal(z, z2)
        assert torch.isfinite(z.float()).all()
