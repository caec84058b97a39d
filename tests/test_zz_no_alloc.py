"""sqattn_quantize_qk_noalloc (the allocation-free form of sqattn_quantize_qk,
for callers that cannot allocate memory) against sqattn_quantize_qk, through
the C-ABI: codes, scales and the K mean equal bit for bit on two calls in a
row, the second on a smaller input (the static scratch keeps the first call's
contents, which the second must not depend on); sizes beyond the scratch are
refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu

WORKSPACE = 3


def _direct(Q, K, q_block):
    """sqattn_quantize_qk_noalloc through its C symbol on torch-allocated outputs."""
    B, H, N, d = Q.shape
    qi = torch.empty((B, H, N, d), dtype=torch.int8, device="cuda")
    ki = torch.empty_like(qi)
    qs = torch.empty((B, H, -(-N // q_block)), dtype=torch.float32, device="cuda")
    ks = torch.empty((B, H, -(-N // 64)), dtype=torch.float32, device="cuda")
    mu = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    for t in (qi, ki, qs, ks, mu):
        t.fill_(-7)   # leftovers must not survive
    st = torch.cuda.current_stream().cuda_stream
    rc = sq.lib().sqattn_quantize_qk_noalloc(Q.data_ptr(), K.data_ptr(), B, H, N, d, q_block, 64, qi.data_ptr(),
                                             qs.data_ptr(), ki.data_ptr(), ks.data_ptr(), mu.data_ptr(), st)
    assert rc == 0, sq.lib().sqattn_last_error()
    return qi, qs, ki, ks, mu


@pytest.mark.parametrize("first,second", [((2, 8, 40000, 128), (1, 3, 700, 64)),
                                          ((1, 40, 32760, 128), (1, 2, 1000, 128))])
def test_noalloc_equals_quantize_qk_twice(first, second):
    for (B, H, N, d), q_block in ((first, 128), (second, 64)):
        w = W.get("wan14b-480p")
        q, k, _, _ = W.gen_inputs(w, N=N, d=d, B=B, H=H)
        Q, K = dev_bf16(q), dev_bf16(k)
        print(f"case B={B} H={H} N={N} d={d} q_block={q_block}", flush=True)
        ref = sq.quantize_qk(Q, K, q_block, 64)
        got = _direct(Q, K, q_block)
        torch.cuda.synchronize()
        for a, b, n in zip(got, ref, ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean")):
            assert torch.equal(a.view(torch.int8) if a.dtype == torch.int8 else a.view(torch.int32),
                               b.view(torch.int8) if b.dtype == torch.int8 else b.view(torch.int32)), n
    # the binding's wrapper reaches the same entry point
    got = sq.quantize_qk_noalloc(Q, K, q_block, 64)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    # 65535 heads need ~268 MB of K-mean partial sums: refused, nothing enqueued
    L = sq.lib()
    need = L.sqattn_quantize_qk_workspace_bytes(1, 65535, 512, 128)
    assert need > (16 << 20)
    fake = 0x100000
    rc = L.sqattn_quantize_qk_noalloc(fake, fake, 1, 65535, 512, 128, 128, 64, fake, fake, fake, fake, fake, None)
    assert rc == WORKSPACE
    assert "static scratch" in L.sqattn_last_error().decode()
