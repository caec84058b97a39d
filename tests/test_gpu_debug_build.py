"""The checking build (libsqattn_debug.so, include/sqattn_debug.h) against
the release build on the GPU: bit-identical outputs (the checking build
drains every load in flight before each work-group barrier, so a wait the
release build's ring schedule is missing would show up as a difference) and
no failed index check, over both P.V types, ragged lengths, d = 64 and 128,
block-sparse masks and Q smoothing."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu

_dbg = None


def _debug_lib():
    global _dbg
    if _dbg is None:
        L = sq.load_library(sq.debug_lib_path)
        L.sqattn_debug_violations.restype = ctypes.c_uint32
        L.sqattn_debug_violations.argtypes = []
        _dbg = L
    return _dbg


def _forward(L, Q, K, V, scale, pv, q_block, smooth, mask):
    B, H, N, d = Q.shape
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device)
    o = sq.Opts(q_block=q_block, k_block=64, v_block=64, out_dtype=0, smooth_q=int(smooth), second_pass_count=None)
    wb = int(L.sqattn_workspace_bytes(B, H, N, d, sq._PV[pv], ctypes.byref(o)))
    ws = torch.empty(wb, dtype=torch.uint8, device=Q.device)
    stream = torch.cuda.current_stream().cuda_stream
    if mask is None:
        st = L.sqattn_forward_ex(Q.data_ptr(), K.data_ptr(), V.data_ptr(), B, H, N, d, float(scale), sq._PV[pv],
                                 out.data_ptr(), ws.data_ptr(), wb, stream, ctypes.byref(o))
    else:
        st = L.sqattn_forward_sparse(Q.data_ptr(), K.data_ptr(), V.data_ptr(), B, H, N, d, float(scale),
                                     sq._PV[pv], mask.data_ptr(), out.data_ptr(), ws.data_ptr(), wb, stream,
                                     ctypes.byref(o))
    assert st == 0, L.sqattn_last_error().decode()
    return out


@pytest.mark.parametrize("case", [
    dict(idx=1, N=700, d=128, H=3, pv="bf16"),
    dict(idx=3, N=700, d=128, H=2, pv="fp8"),
    dict(idx=1, N=65, d=64, H=2, pv="bf16"),
    dict(idx=3, N=63, d=64, H=2, pv="fp8"),
    dict(idx=2, N=4097, d=128, H=2, pv="bf16"),
    dict(idx=3, N=2000, d=128, H=2, pv="fp8", q_block=1),
    dict(idx=1, N=1000, d=128, H=2, pv="bf16", density=0.3),
    dict(idx=3, N=1000, d=128, H=2, pv="fp8", density=0.3),
    dict(idx=1, N=777, d=128, H=2, pv="bf16", smooth=True),
    dict(idx=3, N=777, d=128, H=2, pv="fp8", smooth=True),
])
def test_checking_build_equals_release(case):
    w = W.get(case["idx"])
    q, k, v, _ = W.gen_inputs(w, N=case["N"], d=case["d"], B=1, H=case["H"])
    if case.get("smooth"):
        q = W.add_channel_offset(q, 4.0, seed=9)
    print(f"case {case}", flush=True)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    mask = None
    if "density" in case:
        mask = torch.from_numpy(W.gen_block_mask(1, case["H"], case["N"], case["density"], seed=3)).cuda()
    args = (Q, K, V, w.scale, case["pv"], case.get("q_block", 128), case.get("smooth", False), mask)
    D = _debug_lib()
    assert D.sqattn_debug_violations() == 0
    ref = _forward(sq.lib(), *args)
    out = _forward(D, *args)
    torch.cuda.synchronize()
    assert D.sqattn_debug_violations() == 0
    assert torch.equal(out, ref), float((out - ref).abs().max())


def test_checking_build_full_grid():
    # a full Wan-14B-480p-sized grid in both builds, both P.V types
    w = W.get(2)
    q, k, v, _ = W.gen_inputs(w, H=8)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    D = _debug_lib()
    assert D.sqattn_debug_violations() == 0
    for pv in ("bf16", "fp8"):
        print(f"full grid {pv}", flush=True)
        ref = _forward(sq.lib(), Q, K, V, w.scale, pv, 128, False, None)
        out = _forward(D, Q, K, V, w.scale, pv, 128, False, None)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), pv
    assert D.sqattn_debug_violations() == 0
