"""Python binding of libsqattn (low-bit quantized attention on MI355X / gfx950).

Argument marshalling only: every step runs in the library's HIP kernels behind
the C-ABI declared in ``include/sqattn.h``.  PyTorch provides device memory and
the current stream.  If ``libsqattn.so`` is missing the binding raises; there
is no other implementation to fall back on.

    import bit_quantized_attention_block_amd as sq
    out = sq.forward(q, k, v)                  # bf16 [B,H,N,d] cuda tensors -> fp32
    qi, qs, ki, ks, mu = sq.quantize_qk(q, k)  # INT8 codes, scales, K mean
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["lib", "lib_path", "SqattnError", "quantize_qk", "quantize_qk_noalloc", "quantize_v_fp8", "forward",
           "attend_quantized", "attend_packed", "pack_v", "workspace_bytes", "packed_v_bytes",
           "quantize_qk_workspace_bytes", "PV_BF16", "PV_FP8", "version", "EXPORTS",
           "w8a8_quantize", "w8a8_gemm", "w8a8_linear", "w8a8_workspace_bytes", "w8a8_rmsnorm_quantize",
           "w8a8_linear_rmsnorm", "w8a8_rmsnorm_workspace_bytes", "forward_qknorm",
           "forward_qknorm_workspace_bytes", "w8a8_layernorm_quantize", "w8a8_layernorm_workspace_bytes",
           "w8a8_linear_layernorm"]

PV_BF16 = 0
PV_FP8 = 1
_PV = {"bf16": PV_BF16, "fp8": PV_FP8, PV_BF16: PV_BF16, PV_FP8: PV_FP8}

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libsqattn.so")
# the checking build (include/sqattn_debug.h): same C-ABI, for tests
debug_lib_path = os.path.join(_HERE, "libsqattn_debug.so")

_c = ctypes
_vp, _i, _f, _sz = _c.c_void_p, _c.c_int, _c.c_float, _c.c_size_t

# name -> (restype, argtypes); mirrors include/sqattn.h
EXPORTS = {
    "sqattn_version": (_i, []),
    "sqattn_status_string": (_c.c_char_p, [_i]),
    "sqattn_last_error": (_c.c_char_p, []),
    "sqattn_quantize_qk_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "sqattn_quantize_qk": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sqattn_quantize_qk_noalloc": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sqattn_quantize_v_fp8": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "sqattn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _vp]),
    "sqattn_forward": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _sz, _vp]),
    "sqattn_forward_ex": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _sz, _vp, _vp]),
    "sqattn_packed_v_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "sqattn_pack_v": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "sqattn_attend_quantized": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp,
                                     _vp]),
    "sqattn_attend_packed": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp]),
    "sqattn_forward_sparse": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _sz, _vp, _vp]),
    "sqattn_forward_strided": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _f, _i, _vp, _vp, _vp, _sz, _vp,
                                    _vp]),
    "sqattn_forward_qknorm_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _vp]),
    "sqattn_forward_qknorm": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _i, _vp, _vp, _vp,
                                   _sz, _vp, _vp]),
    "sqattn_attend_quantized_sparse": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp,
                                            _vp, _vp]),
    "sqattn_attend_packed_sparse": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp,
                                         _vp]),
    "sqattn_w8a8_quantize": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "sqattn_w8a8_gemm": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "sqattn_w8a8_workspace_bytes": (_sz, [_i, _i]),
    "sqattn_w8a8_linear": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "sqattn_w8a8_rmsnorm_quantize": (_i, [_vp, _vp, _f, _i, _i, _vp, _vp, _vp, _vp]),
    "sqattn_w8a8_rmsnorm_workspace_bytes": (_sz, [_i, _i]),
    "sqattn_w8a8_linear_rmsnorm": (_i, [_vp, _vp, _f, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "sqattn_w8a8_layernorm_quantize": (_i, [_vp, _vp, _vp, _f, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "sqattn_w8a8_layernorm_workspace_bytes": (_sz, [_i, _i]),
    "sqattn_w8a8_linear_layernorm": (_i, [_vp, _vp, _vp, _f, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
}


class Opts(ctypes.Structure):
    _fields_ = [("q_block", _i), ("k_block", _i), ("v_block", _i), ("out_dtype", _i), ("smooth_q", _i),
                ("second_pass_count", ctypes.c_void_p)]


class SqattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sqattn status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: str):
    """A ctypes.CDLL of a libsqattn build at `path` with the C-ABI's argument
    and result types set (the binding's own library is lib())."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bit_quantized_attention_block_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """The loaded libsqattn (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(lib_path)
    return _lib


def version() -> int:
    return lib().sqattn_version()


def _check(status: int):
    if status != 0:
        L = lib()
        raise SqattnError(status, f"{L.sqattn_status_string(status).decode()}: "
                                  f"{L.sqattn_last_error().decode()}")


# --------------------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _shape(q):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


def _ws(nbytes, device, workspace):
    torch = _torch()
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        return workspace, workspace.numel()
    if nbytes == 0:
        return None, 0
    w = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return w, nbytes


# --------------------------------------------------------------------------- API

def quantize_qk_workspace_bytes(B, H, N, d) -> int:
    return int(lib().sqattn_quantize_qk_workspace_bytes(B, H, N, d))


def quantize_qk(q, k, q_block: int = 128, k_block: int = 64, workspace=None):
    """Q, K bf16 [B,H,N,d] -> (q_i8, q_scale, k_i8, k_scale, k_mean)."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16)
    B, H, N, d = _shape(q)
    if tuple(k.shape) != (B, H, N, d):
        raise ValueError("q and k shapes differ")
    dev = q.device
    qi = torch.empty((B, H, N, d), dtype=torch.int8, device=dev)
    ki = torch.empty_like(qi)
    qs = torch.empty((B, H, -(-N // q_block)), dtype=torch.float32, device=dev)
    ks = torch.empty((B, H, -(-N // k_block)), dtype=torch.float32, device=dev)
    mu = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    w, wb = _ws(quantize_qk_workspace_bytes(B, H, N, d), dev, workspace)
    _check(lib().sqattn_quantize_qk(_ptr(q), _ptr(k), B, H, N, d, q_block, k_block, _ptr(qi), _ptr(qs),
                                    _ptr(ki), _ptr(ks), _ptr(mu), _ptr(w), wb, _stream(q)))
    return qi, qs, ki, ks, mu


def quantize_qk_noalloc(q, k, q_block: int = 128, k_block: int = 64, outs=None):
    """quantize_qk through sqattn_quantize_qk_noalloc: the library allocates
    nothing (the K-mean partial sums live in its static device scratch).
    outs: the caller's (q_i8, q_scale, k_i8, k_scale, k_mean) tensors, or None
    to have them allocated here by torch."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16)
    B, H, N, d = _shape(q)
    if tuple(k.shape) != (B, H, N, d):
        raise ValueError("q and k shapes differ")
    dev = q.device
    if outs is None:
        outs = (torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
                torch.empty((B, H, -(-N // q_block)), dtype=torch.float32, device=dev),
                torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
                torch.empty((B, H, -(-N // k_block)), dtype=torch.float32, device=dev),
                torch.empty((B, H, d), dtype=torch.float32, device=dev))
    qi, qs, ki, ks, mu = outs
    for t, n, dt, shape in ((qi, "q_i8", torch.int8, (B, H, N, d)), (ki, "k_i8", torch.int8, (B, H, N, d)),
                            (qs, "q_scale", torch.float32, (B, H, -(-N // q_block))),
                            (ks, "k_scale", torch.float32, (B, H, -(-N // k_block))),
                            (mu, "k_mean", torch.float32, (B, H, d))):
        _dev(t, n, dt)
        if tuple(t.shape) != shape:
            raise ValueError(f"{n} must have shape {shape}")
    _check(lib().sqattn_quantize_qk_noalloc(_ptr(q), _ptr(k), B, H, N, d, q_block, k_block, _ptr(qi), _ptr(qs),
                                            _ptr(ki), _ptr(ks), _ptr(mu), _stream(q)))
    return qi, qs, ki, ks, mu


def quantize_v_fp8(v, v_block: int = 64):
    """V bf16 [B,H,N,d] -> (E4M3 codes uint8 [B,H,N,d], scales [B,H,ceil(N/64)])."""
    torch = _torch()
    _dev(v, "v", torch.bfloat16)
    B, H, N, d = _shape(v)
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=v.device)
    sc = torch.empty((B, H, -(-N // v_block)), dtype=torch.float32, device=v.device)
    _check(lib().sqattn_quantize_v_fp8(_ptr(v), B, H, N, d, v_block, _ptr(codes), _ptr(sc), _stream(v)))
    return codes, sc


OUT_FP32, OUT_BF16 = 0, 1


def _opts(q_block, out_dtype=OUT_FP32, second_pass_count=None, smooth_q=False):
    """sqattn_opts; second_pass_count: None or a one-element int32 device
    tensor the 16-bit P.V kernel increments per (head, 256-row block) that
    took the exact-max second pass (the caller zeroes it); smooth_q: Q
    smoothing per Q block (forward only)."""
    c = None
    if second_pass_count is not None:
        torch = _torch()
        _dev(second_pass_count, "second_pass_count", torch.int32)
        if second_pass_count.numel() < 1:
            raise ValueError("second_pass_count must hold one element")
        c = second_pass_count.data_ptr()
    return Opts(q_block=int(q_block), k_block=64, v_block=64, out_dtype=out_dtype, smooth_q=int(bool(smooth_q)),
                second_pass_count=c)


def _out(out, shape, dev, out_dtype):
    """The output tensor (allocated when None) and its sqattn_out_dtype code:
    fp32 by default, bf16 (the fp32 result rounded to nearest even) when
    out_dtype is torch.bfloat16 or a bf16 `out` is given."""
    torch = _torch()
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"out_dtype must be torch.float32 or torch.bfloat16, got {out_dtype}")
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    _dev(out, "out", out_dtype)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out, (OUT_BF16 if out_dtype == torch.bfloat16 else OUT_FP32)


def workspace_bytes(B, H, N, d, pv="bf16", q_block: int = 128, smooth_q: bool = False) -> int:
    o = _opts(q_block, smooth_q=smooth_q)
    return int(lib().sqattn_workspace_bytes(B, H, N, d, _PV[pv], ctypes.byref(o)))


def _mask(block_mask, B, H, N):
    """The block mask as a contiguous uint8 device tensor [B,H,ceil(N/128),ceil(N/64)]."""
    torch = _torch()
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    _dev(block_mask, "block_mask", torch.uint8)
    want = (B, H, -(-N // 128), -(-N // 64))
    if tuple(block_mask.shape) != want:
        raise ValueError(f"block_mask has shape {tuple(block_mask.shape)}, expected {want}")
    return block_mask


def _row_strides(t, name, dtype):
    """(b, h, n) element strides of a [B,H,N,d] device tensor whose rows are
    contiguous (a view, e.g. of a fused QKV projection output)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be [B,H,N,d] with contiguous rows")
    return tuple(int(x) for x in t.stride()[:3])


def forward(q, k, v, scale: float | None = None, pv="bf16", q_block: int = 128, out=None,
            workspace=None, out_dtype=None, block_mask=None, second_pass_count=None, smooth_q: bool = False):
    """Quantized attention forward: bf16 q, k, v [B,H,N,d] -> out [B,H,N,d],
    fp32 or (out_dtype=torch.bfloat16, or a bf16 `out`) bf16.  block_mask
    (uint8/bool [B,H,ceil(N/128),ceil(N/64)]): block-sparse attention over
    the kept (128-row query block, 64-key tile) pairs.  q, k, v and out may be
    strided views with contiguous rows (e.g. q = qkv[:, :, 0].transpose(1, 2)
    of a [B,N,3,H,d] projection output); they go through
    sqattn_forward_strided.  second_pass_count, smooth_q (Q smoothing per Q
    block, q_block 64, 128 or 256, dense): see _opts."""
    torch = _torch()
    strided = any(isinstance(t, torch.Tensor) and not t.is_contiguous() for t in (q, k, v, out))
    if strided:
        return _forward_strided(q, k, v, scale, pv, q_block, out, workspace, out_dtype, block_mask,
                                second_pass_count=second_pass_count, smooth_q=smooth_q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, torch.bfloat16)
    B, H, N, d = _shape(q)
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v shapes differ")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, od = _out(out, (B, H, N, d), q.device, out_dtype)
    w, wb = _ws(workspace_bytes(B, H, N, d, pv, q_block, smooth_q), q.device, workspace)
    o = _opts(q_block, od, second_pass_count, smooth_q)
    if block_mask is not None:
        m = _mask(block_mask, B, H, N)
        _check(lib().sqattn_forward_sparse(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), _PV[pv], _ptr(m),
                                           _ptr(out), _ptr(w), wb, _stream(q), ctypes.byref(o)))
        return out
    if q_block == 128 and od == OUT_FP32 and second_pass_count is None and not smooth_q:
        # the default options: the plain entry point (q_block 128, k/v blocks 64, fp32 out)
        _check(lib().sqattn_forward(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), _PV[pv], _ptr(out),
                                    _ptr(w), wb, _stream(q)))
        return out
    _check(lib().sqattn_forward_ex(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), _PV[pv], _ptr(out),
                                   _ptr(w), wb, _stream(q), ctypes.byref(o)))
    return out


def forward_qknorm_workspace_bytes(B, H, N, d, pv="bf16", q_block: int = 128) -> int:
    o = _opts(q_block, OUT_FP32)
    return int(lib().sqattn_forward_qknorm_workspace_bytes(B, H, N, d, _PV[pv], ctypes.byref(o)))


def forward_qknorm(q, k, v, gamma_q=None, gamma_k=None, eps: float = 1e-6, scale: float | None = None, pv="bf16",
                   q_block: int = 128, out=None, workspace=None, out_dtype=None, block_mask=None,
                   second_pass_count=None):
    """Attention with the per-token RMSNorm of q and k (over each token's H*d
    features, weights gamma_q / gamma_k fp32 [H*d] or None) fused into their
    quantization; sqattn_forward_qknorm.  q, k, v: bf16 [B,H,N,d] views whose
    q and k head stride is d (e.g. slices of a fused [B,N,3,H,d] projection
    output, permuted)."""
    torch = _torch()
    for g, n in ((gamma_q, "gamma_q"), (gamma_k, "gamma_k")):
        if g is not None:
            _dev(g, n, torch.float32)
            if g.numel() != q.shape[1] * q.shape[3]:
                raise ValueError(f"{n} has {g.numel()} elements, expected H*d = {q.shape[1] * q.shape[3]}")
    return _forward_strided(q, k, v, scale, pv, q_block, out, workspace, out_dtype, block_mask,
                            qkn=(gamma_q, gamma_k, float(eps)), second_pass_count=second_pass_count)


def _forward_strided(q, k, v, scale, pv, q_block, out, workspace, out_dtype, block_mask, qkn=None,
                     second_pass_count=None, smooth_q=False):
    torch = _torch()
    st = []
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        st += _row_strides(t, n, torch.bfloat16)
    B, H, N, d = _shape(q)
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v shapes differ")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    if tuple(out.shape) != (B, H, N, d):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(B, H, N, d)}")
    ost = _row_strides(out, "out", out_dtype)
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_FP32
    o = _opts(q_block, od, second_pass_count, smooth_q)
    m = _mask(block_mask, B, H, N) if block_mask is not None else None
    ins = (ctypes.c_int64 * 9)(*st)
    outs = (ctypes.c_int64 * 3)(*ost)
    if qkn is None:
        w, wb = _ws(workspace_bytes(B, H, N, d, pv, q_block, smooth_q), q.device, workspace)
        _check(lib().sqattn_forward_strided(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, ins, outs, float(scale),
                                            _PV[pv], _ptr(m), _ptr(out), _ptr(w), wb, _stream(q), ctypes.byref(o)))
    else:
        w, wb = _ws(forward_qknorm_workspace_bytes(B, H, N, d, pv, q_block), q.device, workspace)
        gq, gk, eps = qkn
        _check(lib().sqattn_forward_qknorm(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, ins, outs, _ptr(gq), _ptr(gk),
                                           eps, float(scale), _PV[pv], _ptr(m), _ptr(out), _ptr(w), wb,
                                           _stream(q), ctypes.byref(o)))
    return out


def packed_v_bytes(B, H, N, d, pv="bf16") -> int:
    return int(lib().sqattn_packed_v_bytes(B, H, N, d, _PV[pv]))


def pack_v(v, pv="bf16"):
    """bf16 V (pv="bf16") or E4M3 V codes (pv="fp8") [B,H,N,d] -> the attention
    kernel's tile layout (a flat uint8 tensor)."""
    torch = _torch()
    _dev(v, "v", torch.bfloat16 if _PV[pv] == PV_BF16 else torch.uint8)
    B, H, N, d = _shape(v)
    packed = torch.empty(packed_v_bytes(B, H, N, d, pv), dtype=torch.uint8, device=v.device)
    _check(lib().sqattn_pack_v(_ptr(v), B, H, N, d, _PV[pv], _ptr(packed), _stream(v)))
    return packed


def _attend(packed, q_i8, q_scale, k_i8, k_scale, v, v_scale, scale, pv, q_block, out, out_dtype, block_mask,
            second_pass_count=None):
    torch = _torch()
    _dev(q_i8, "q_i8", torch.int8)
    _dev(k_i8, "k_i8", torch.int8)
    _dev(q_scale, "q_scale", torch.float32)
    _dev(k_scale, "k_scale", torch.float32)
    B, H, N, d = _shape(q_i8)
    if packed:
        _dev(v, "v_packed", torch.uint8)
        if v.numel() < packed_v_bytes(B, H, N, d, pv):
            raise ValueError("v_packed is too small")
    else:
        _dev(v, "v", torch.bfloat16 if _PV[pv] == PV_BF16 else torch.uint8)
        if _shape(v) != (B, H, N, d):
            raise ValueError("v must have the shape of q_i8")
    if _PV[pv] == PV_FP8:
        _dev(v_scale, "v_scale", torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, od = _out(out, (B, H, N, d), q_i8.device, out_dtype)
    o = _opts(q_block, od, second_pass_count)
    L = lib()
    args = (_ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(v), _ptr(v_scale), B, H, N, d,
            float(scale), _PV[pv])
    if block_mask is not None:
        m = _mask(block_mask, B, H, N)
        fn = L.sqattn_attend_packed_sparse if packed else L.sqattn_attend_quantized_sparse
        _check(fn(*args, _ptr(m), ctypes.byref(o), _ptr(out), _stream(q_i8)))
        return out
    fn = L.sqattn_attend_packed if packed else L.sqattn_attend_quantized
    _check(fn(*args, ctypes.byref(o), _ptr(out), _stream(q_i8)))
    return out


def attend_quantized(q_i8, q_scale, k_i8, k_scale, v, v_scale=None, scale: float | None = None,
                     pv="bf16", q_block: int = 128, out=None, out_dtype=None, block_mask=None,
                     second_pass_count=None):
    """Attention on quantized Q/K (from quantize_qk) and V: bf16 [B,H,N,d] for
    pv="bf16", E4M3 codes (from quantize_v_fp8) with their scales for
    pv="fp8"; block_mask as in forward."""
    return _attend(False, q_i8, q_scale, k_i8, k_scale, v, v_scale, scale, pv, q_block, out, out_dtype,
                   block_mask, second_pass_count)


def attend_packed(q_i8, q_scale, k_i8, k_scale, v_packed, v_scale=None, scale: float | None = None,
                  pv="bf16", q_block: int = 128, out=None, out_dtype=None, block_mask=None,
                  second_pass_count=None):
    """The attention kernel alone, on quantized Q/K and V already in the
    kernel's tile layout (see pack_v)."""
    return _attend(True, q_i8, q_scale, k_i8, k_scale, v_packed, v_scale, scale, pv, q_block, out, out_dtype,
                   block_mask, second_pass_count)


# --------------------------------------------------------------------------- W8A8 linear

def w8a8_quantize(x):
    """bf16 [R, K] (K a multiple of 128) -> (int8 codes [R, K], float32
    scales [ceil(R/128), K/128]), one scale per 128x128 block."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    R, C = (int(v) for v in x.shape)
    codes = torch.empty((R, C), dtype=torch.int8, device=x.device)
    scales = torch.empty((-(-R // 128), C // 128 if C % 128 == 0 else 0), dtype=torch.float32, device=x.device)
    _check(lib().sqattn_w8a8_quantize(_ptr(x), R, C, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def _w8a8_shapes(x_shape, w_codes, w_scales, bias):
    torch = _torch()
    _dev(w_codes, "w_codes", torch.int8)
    _dev(w_scales, "w_scales", torch.float32)
    if w_codes.dim() != 2:
        raise ValueError("w_codes must be [N, K]")
    M, K = (int(v) for v in x_shape)
    N, K2 = (int(v) for v in w_codes.shape)
    if K != K2:
        raise ValueError(f"x has K = {K}, w_codes has K = {K2}")
    if K % 128 == 0 and tuple(w_scales.shape) != (-(-N // 128), K // 128):
        raise ValueError("w_scales must be [ceil(N/128), K/128]")
    if bias is not None:
        _dev(bias, "bias", torch.float32)
        if tuple(bias.shape) != (N,):
            raise ValueError("bias must be [N]")
    return M, N, K


def w8a8_gemm(x_codes, x_scales, w_codes, w_scales, bias=None, out=None, out_dtype=None):
    """y = x W^T (+ bias) from block codes and scales (see w8a8_quantize):
    [M, N] fp32, or bf16 (out_dtype=torch.bfloat16 or a bf16 `out`)."""
    torch = _torch()
    _dev(x_codes, "x_codes", torch.int8)
    _dev(x_scales, "x_scales", torch.float32)
    if x_codes.dim() != 2:
        raise ValueError("x_codes must be [M, K]")
    M, N, K = _w8a8_shapes(x_codes.shape, w_codes, w_scales, bias)
    if K % 128 == 0 and tuple(x_scales.shape) != (-(-M // 128), K // 128):
        raise ValueError("x_scales must be [ceil(M/128), K/128]")
    out, od = _out(out, (M, N), x_codes.device, out_dtype)
    _check(lib().sqattn_w8a8_gemm(_ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scales), _ptr(bias),
                                  M, N, K, od, _ptr(out), _stream(x_codes)))
    return out


def w8a8_workspace_bytes(M, K) -> int:
    return int(lib().sqattn_w8a8_workspace_bytes(M, K))


def w8a8_linear(x, w_codes, w_scales, bias=None, out=None, out_dtype=None, workspace=None):
    """The W8A8 layer on bf16 activations x [M, K] and pre-quantized weights
    (w8a8_quantize of W [N, K]): quantizes x, then the block-scaled GEMM."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, N, K = _w8a8_shapes(x.shape, w_codes, w_scales, bias)
    out, od = _out(out, (M, N), x.device, out_dtype)
    w, wb = _ws(w8a8_workspace_bytes(M, K), x.device, workspace)
    _check(lib().sqattn_w8a8_linear(_ptr(x), _ptr(w_codes), _ptr(w_scales), _ptr(bias), M, N, K, od, _ptr(out),
                                    _ptr(w), wb, _stream(x)))
    return out


def _gamma(gamma, K):
    torch = _torch()
    if gamma is None:
        return None
    _dev(gamma, "gamma", torch.float32)
    if tuple(gamma.shape) != (K,):
        raise ValueError(f"gamma must be [{K}]")
    return gamma


def w8a8_rmsnorm_workspace_bytes(M, K) -> int:
    return int(lib().sqattn_w8a8_rmsnorm_workspace_bytes(M, K))


def w8a8_rmsnorm_quantize(x, gamma=None, eps: float = 1e-6):
    """RMSNorm of bf16 x [R, K] (gamma fp32 [K] or None) fused with the W8A8
    block quantization: (codes, scales, inv_rms [R])."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    R, C = (int(v) for v in x.shape)
    codes = torch.empty((R, C), dtype=torch.int8, device=x.device)
    scales = torch.empty((-(-R // 128), C // 128 if C % 128 == 0 else 0), dtype=torch.float32, device=x.device)
    r = torch.empty((R,), dtype=torch.float32, device=x.device)
    g = _gamma(gamma, C)
    _check(lib().sqattn_w8a8_rmsnorm_quantize(_ptr(x), _ptr(g), float(eps), R, C, _ptr(codes), _ptr(scales), _ptr(r),
                                              _stream(x)))
    return codes, scales, r


def w8a8_linear_rmsnorm(x, w_codes, w_scales, gamma=None, eps: float = 1e-6, bias=None, out=None, out_dtype=None,
                        workspace=None):
    """RMSNorm(x) W^T (+ bias): the normalization, the INT8 block quantization
    and the block-scaled GEMM, with no normalized activations in HBM."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, N, K = _w8a8_shapes(x.shape, w_codes, w_scales, bias)
    g = _gamma(gamma, K)
    out, od = _out(out, (M, N), x.device, out_dtype)
    w, wb = _ws(w8a8_rmsnorm_workspace_bytes(M, K), x.device, workspace)
    _check(lib().sqattn_w8a8_linear_rmsnorm(_ptr(x), _ptr(g), float(eps), _ptr(w_codes), _ptr(w_scales), _ptr(bias),
                                            M, N, K, od, _ptr(out), _ptr(w), wb, _stream(x)))
    return out


def w8a8_layernorm_workspace_bytes(M, K) -> int:
    return int(lib().sqattn_w8a8_layernorm_workspace_bytes(M, K))


def w8a8_layernorm_quantize(x, gamma=None, beta=None, eps: float = 1e-6):
    """LayerNorm of bf16 x [R, K] (gamma, beta fp32 [K] or None) fused with
    the W8A8 block quantization: (codes, scales, mean [R], rstd [R])."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    R, C = (int(v) for v in x.shape)
    codes = torch.empty((R, C), dtype=torch.int8, device=x.device)
    scales = torch.empty((-(-R // 128), C // 128 if C % 128 == 0 else 0), dtype=torch.float32, device=x.device)
    mu = torch.empty((R,), dtype=torch.float32, device=x.device)
    r = torch.empty((R,), dtype=torch.float32, device=x.device)
    g, b = _gamma(gamma, C), _gamma(beta, C)
    _check(lib().sqattn_w8a8_layernorm_quantize(_ptr(x), _ptr(g), _ptr(b), float(eps), R, C, _ptr(codes),
                                                _ptr(scales), _ptr(mu), _ptr(r), _stream(x)))
    return codes, scales, mu, r


def w8a8_linear_layernorm(x, w_codes, w_scales, gamma=None, beta=None, eps: float = 1e-6, bias=None, out=None,
                          out_dtype=None, workspace=None):
    """LayerNorm(x) W^T (+ bias): normalization, INT8 block quantization and
    the block-scaled GEMM, with no normalized activations in HBM."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, N, K = _w8a8_shapes(x.shape, w_codes, w_scales, bias)
    g, b = _gamma(gamma, K), _gamma(beta, K)
    out, od = _out(out, (M, N), x.device, out_dtype)
    w, wb = _ws(w8a8_layernorm_workspace_bytes(M, K), x.device, workspace)
    _check(lib().sqattn_w8a8_linear_layernorm(_ptr(x), _ptr(g), _ptr(b), float(eps), _ptr(w_codes), _ptr(w_scales),
                                              _ptr(bias), M, N, K, od, _ptr(out), _ptr(w), wb, _stream(x)))
    return out
