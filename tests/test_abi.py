"""CPU tests of the C-ABI library: it loads, exports every symbol that
include/sqattn.h declares (as unmangled C symbols), and rejects bad arguments
with the documented status before anything is enqueued (so no GPU is needed:
every call below returns from host-side validation)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import bit_quantized_attention_block_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "sqattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, RANGE = 0, 1, 2, 3, 4, 5
FAKE = 0x100000          # 256-byte aligned, never dereferenced
BIG = 1 << 40


def declared():
    txt = re.sub(r"/\*.*?\*/", "", open(HDR).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(sqattn_[a-z0-9_]+)\s*\(", txt)))


def test_library_loads_and_exports_every_declared_function():
    L = sq.lib()
    names = declared()
    assert len(names) == 30
    assert set(names) == set(sq.EXPORTS), "binding and header disagree"
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", sq.lib_path], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    for n in names:
        assert n in syms, f"{n} is not an exported C symbol"
    assert sq.version() == 10100


def test_checking_build_exports_the_same_calls_and_its_own():
    # libsqattn_debug.so: every call of include/sqattn.h plus the one of
    # include/sqattn_debug.h
    dbg = os.path.join(ROOT, "include", "sqattn_debug.h")
    txt = re.sub(r"/\*.*?\*/", "", open(dbg).read(), flags=re.S)
    extra = sorted(set(re.findall(r"\b(sqattn_[a-z0-9_]+)\s*\(", txt)))
    assert extra == ["sqattn_debug_violations"]
    nm = subprocess.run(["nm", "-D", "--defined-only", sq.debug_lib_path], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    for n in declared() + extra:
        assert n in syms, n
    rel = subprocess.run(["nm", "-D", "--defined-only", sq.lib_path], capture_output=True, text=True).stdout
    assert "sqattn_debug_violations" not in rel
    L = sq.load_library(sq.debug_lib_path)
    assert L.sqattn_version() == sq.version()


def test_status_strings():
    L = sq.lib()
    for s in range(6):
        assert L.sqattn_status_string(s).decode()
    assert L.sqattn_status_string(99).decode() == "unknown status"


def _fwd(q=FAKE, k=FAKE, v=FAKE, B=1, H=1, N=256, d=64, scale=0.125, pv=0, out=FAKE, ws=FAKE, wsb=1,
         opts=None):
    L = sq.lib()
    o = ctypes.byref(opts) if opts is not None else None
    return L.sqattn_forward_ex(q, k, v, B, H, N, d, scale, pv, out, ws, wsb, None, o)


def _err():
    return sq.lib().sqattn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=None), INVALID, "q is NULL"),
    (dict(v=None), INVALID, "v is NULL"),
    (dict(out=FAKE + 4), INVALID, "aligned"),
    (dict(k=FAKE + 8), INVALID, "aligned"),
    (dict(B=0), INVALID, ">= 1"),
    (dict(N=0), INVALID, ">= 1"),
    (dict(H=-3), INVALID, ">= 1"),
    (dict(d=96), UNSUPPORTED, "64 or 128"),
    (dict(d=256), UNSUPPORTED, "64 or 128"),
    (dict(N=1 << 24), RANGE, "2^24"),
    (dict(B=300, H=300), RANGE, "65535"),
    (dict(pv=2), INVALID, "pv_dtype"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(scale=-1.0), INVALID, "scale"),
    (dict(wsb=1), WORKSPACE, "needed"),
    (dict(ws=FAKE + 16, wsb=BIG), INVALID, "256-byte"),
    (dict(opts=sq.Opts(128, 128, 64, 0)), UNSUPPORTED, "k_block"),
    (dict(opts=sq.Opts(128, 64, 32, 0)), UNSUPPORTED, "v_block"),
    (dict(opts=sq.Opts(24, 64, 64, 0)), INVALID, "q_block"),
    (dict(opts=sq.Opts(128, 64, 64, 2)), INVALID, "out_dtype"),
    (dict(opts=sq.Opts(128, 64, 64, -1)), INVALID, "out_dtype"),
    (dict(opts=sq.Opts(128, 64, 64, 0, 0, FAKE + 2)), INVALID, "second_pass_count"),
    (dict(opts=sq.Opts(128, 64, 64, 0, 2)), INVALID, "smooth_q"),
    (dict(opts=sq.Opts(16, 64, 64, 0, 1)), UNSUPPORTED, "Q smoothing"),
    (dict(opts=sq.Opts(192, 64, 64, 0, 1)), UNSUPPORTED, "Q smoothing"),
    (dict(opts=sq.Opts(1, 64, 64, 0, 1)), UNSUPPORTED, "Q smoothing"),
])
def test_forward_validation(kw, code, needle):
    assert _fwd(**kw) == code
    assert needle in _err()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=None), INVALID, "q is NULL"),
    (dict(out=FAKE + 4), INVALID, "aligned"),
    (dict(d=96), UNSUPPORTED, "64 or 128"),
    (dict(N=1 << 24), RANGE, "2^24"),
    (dict(pv=2), INVALID, "pv_dtype"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(wsb=1), WORKSPACE, "needed"),
])
def test_plain_forward_validation(kw, code, needle):
    # sqattn_forward (q, k, v, B, H, N, d, scale, pv_dtype, out, workspace, bytes, stream):
    # the same checks as the _ex form with default options, before anything is enqueued
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, H=1, N=256, d=64, scale=0.125, pv=0, out=FAKE, ws=FAKE, wsb=1)
    a.update(kw)
    L = sq.lib()
    rc = L.sqattn_forward(a["q"], a["k"], a["v"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["pv"], a["out"],
                          a["ws"], a["wsb"], None)
    assert rc == code
    assert needle in _err()


def test_quantize_validation():
    L = sq.lib()
    args = [FAKE, FAKE, 1, 1, 256, 128, 128, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None]
    a = list(args)
    a[6] = 0
    assert L.sqattn_quantize_qk(*a) == INVALID and "q_block" in _err()
    a = list(args)
    a[7] = 8
    assert L.sqattn_quantize_qk(*a) == INVALID and "k_block" in _err()
    a = list(args)
    a[12] = None
    assert L.sqattn_quantize_qk(*a) == INVALID and "k_mean" in _err()
    a = list(args)
    a[11] = FAKE + 2
    assert L.sqattn_quantize_qk(*a) == INVALID and "k_scale" in _err()
    # workspace present but too small
    assert L.sqattn_quantize_qk(*args) == WORKSPACE
    assert L.sqattn_quantize_v_fp8(FAKE, 1, 1, 256, 128, 32, FAKE, FAKE, None) == UNSUPPORTED
    assert L.sqattn_quantize_v_fp8(None, 1, 1, 256, 128, 64, FAKE, FAKE, None) == INVALID


def test_attend_and_pack_validation():
    # the raw-V entry point validates everything before it allocates its V
    # temporary (so these calls enqueue and allocate nothing), like the packed one
    L = sq.lib()
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 300, 128, 0.1, 1, None, FAKE, None]
    for fn, vname in ((L.sqattn_attend_quantized, "v"), (L.sqattn_attend_packed, "v_packed")):
        a = list(base)
        a[5] = None                                           # fp8 needs v_scale
        assert fn(*a) == INVALID and "v_scale" in _err()
        a = list(base)
        a[11] = 7
        assert fn(*a) == INVALID
        a = list(base)
        a[4] = FAKE + 1
        assert fn(*a) == INVALID and vname in _err()
        a = list(base)
        a[9] = 32
        assert fn(*a) == UNSUPPORTED
        a = list(base)
        a[13] = None
        assert fn(*a) == INVALID and "out" in _err()
        a = list(base)
        a[10] = float("inf")
        assert fn(*a) == INVALID and "scale" in _err()
    assert L.sqattn_pack_v(FAKE, 1, 1, 100, 128, 3, FAKE, None) == INVALID
    assert L.sqattn_pack_v(FAKE, 1, 1, 100, 128, 0, None, None) == INVALID
    assert L.sqattn_pack_v(FAKE, 1, 1, 0, 128, 0, FAKE, None) == INVALID


def test_workspace_sizes():
    L = sq.lib()
    B, H, N, d = 1, 40, 32760, 128
    nt = -(-N // 64)
    wb = L.sqattn_workspace_bytes(B, H, N, d, 0, None)
    assert wb >= 2 * B * H * N * d + B * H * nt * d * 64 * 2
    w8 = L.sqattn_workspace_bytes(B, H, N, d, 1, None)
    assert w8 < wb and w8 >= 2 * B * H * N * d + B * H * nt * d * 64
    assert L.sqattn_workspace_bytes(B, H, N, 96, 0, None) == 0
    assert L.sqattn_workspace_bytes(B, H, N, d, 5, None) == 0
    assert L.sqattn_packed_v_bytes(B, H, N, d, 0) == B * H * nt * d * 64 * 2
    assert L.sqattn_packed_v_bytes(B, H, N, d, 1) == B * H * nt * d * 64
    assert L.sqattn_quantize_qk_workspace_bytes(B, H, N, d) > 0
    assert L.sqattn_quantize_qk_workspace_bytes(0, H, N, d) == 0
    # the size queries do not disturb the last error message
    _fwd(d=96)
    msg = _err()
    L.sqattn_workspace_bytes(0, 0, 0, 0, 0, None)
    assert _err() == msg


def test_binding_rejects_non_gpu_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sq.forward(q, q, q)
    with pytest.raises(TypeError, match="torch.Tensor"):
        sq.quantize_qk([1.0], q)


def _gemm(xc=FAKE, xs=FAKE, wc=FAKE, ws=FAKE, bias=None, M=300, N=200, K=384, od=0, out=FAKE):
    return sq.lib().sqattn_w8a8_gemm(xc, xs, wc, ws, bias, M, N, K, od, out, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(xc=None), INVALID, "x_codes is NULL"),
    (dict(ws=None), INVALID, "w_scales is NULL"),
    (dict(out=FAKE + 8), INVALID, "aligned"),
    (dict(bias=FAKE + 2), INVALID, "bias"),
    (dict(K=100), INVALID, "multiple of 128"),
    (dict(K=0), INVALID, "multiple of 128"),
    (dict(K=-128), INVALID, "multiple of 128"),
    (dict(K=(1 << 20) + 128), RANGE, "2^20"),
    (dict(M=-1), INVALID, "M must be >= 0"),
    (dict(N=-5), INVALID, "N must be >= 0"),
    (dict(M=65535 * 128 + 1), RANGE, "65535*128"),
    (dict(od=2), INVALID, "out_dtype"),
    (dict(od=-1), INVALID, "out_dtype"),
])
def test_w8a8_gemm_validation(kw, code, needle):
    assert _gemm(**kw) == code
    assert needle in _err()


def test_w8a8_empty_shapes_enqueue_nothing():
    # M = 0 or N = 0 is a valid empty product: OK without touching the GPU
    assert _gemm(M=0) == OK
    assert _gemm(N=0) == OK
    L = sq.lib()
    assert L.sqattn_w8a8_quantize(FAKE, 0, 256, FAKE, FAKE, None) == OK
    assert L.sqattn_w8a8_linear(FAKE, FAKE, FAKE, None, 0, 64, 256, 0, FAKE, None, 0, None) == OK
    # and the pointers of an empty product are not inspected
    assert L.sqattn_w8a8_linear(None, None, None, None, 0, 64, 256, 0, None, None, 0, None) == OK
    assert L.sqattn_w8a8_gemm(None, None, None, None, None, 5, 0, 128, 0, None, None) == OK
    assert L.sqattn_w8a8_quantize(None, 0, 128, None, None, None) == OK
    # sizes are still validated
    assert L.sqattn_w8a8_linear(None, None, None, None, 0, 64, 100, 0, None, None, 0, None) == INVALID


def test_w8a8_quantize_and_linear_validation():
    L = sq.lib()
    assert L.sqattn_w8a8_quantize(FAKE, 10, 200, FAKE, FAKE, None) == INVALID and "128" in _err()
    assert L.sqattn_w8a8_quantize(FAKE + 2, 10, 256, FAKE, FAKE, None) == INVALID and "x is not" in _err()
    assert L.sqattn_w8a8_quantize(FAKE, 10, 256, FAKE, None, None) == INVALID and "scales" in _err()
    assert L.sqattn_w8a8_quantize(FAKE, -1, 256, FAKE, FAKE, None) == INVALID
    lin = [FAKE, FAKE, FAKE, None, 300, 200, 384, 0, FAKE, FAKE, 1, None]
    assert L.sqattn_w8a8_linear(*lin) == WORKSPACE and "needed" in _err()
    a = list(lin)
    a[9] = FAKE + 16
    a[10] = BIG
    assert L.sqattn_w8a8_linear(*a) == INVALID and "256-byte" in _err()
    a = list(lin)
    a[6] = 130
    assert L.sqattn_w8a8_linear(*a) == INVALID


def test_w8a8_workspace_bytes():
    L = sq.lib()
    M, K = 32760, 5120
    need = L.sqattn_w8a8_workspace_bytes(M, K)
    assert need >= M * K + (-(-M // 128)) * (K // 128) * 4 and need % 256 == 0
    assert L.sqattn_w8a8_workspace_bytes(M, 100) == 0
    assert L.sqattn_w8a8_workspace_bytes(-1, K) == 0
    assert L.sqattn_w8a8_workspace_bytes(0, K) == 0 or L.sqattn_w8a8_workspace_bytes(0, K) < 1024


def test_sparse_validation():
    L = sq.lib()
    args = [FAKE, FAKE, FAKE, 1, 1, 256, 64, 0.125, 0, FAKE, FAKE, FAKE, 1, None, None]
    a = list(args)
    a[9] = None
    assert L.sqattn_forward_sparse(*a) == INVALID and "block_mask" in _err()
    a = list(args)
    a[5] = 262144 + 1
    a[12] = BIG
    assert L.sqattn_forward_sparse(*a) == UNSUPPORTED and "262144" in _err()
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 2, 300, 128, 0.1, 0, FAKE, None, FAKE, None]
    for fn in (L.sqattn_attend_quantized_sparse, L.sqattn_attend_packed_sparse):
        a = list(base)
        a[12] = None
        assert fn(*a) == INVALID and "block_mask" in _err()
        a = list(base)
        a[8] = 262144 + 64
        assert fn(*a) == UNSUPPORTED


def test_per_row_q_block_accepted():
    # q_block = 1 passes validation (the call then stops at the workspace size)
    assert _fwd(opts=sq.Opts(1, 64, 64, 0)) == WORKSPACE
    assert _fwd(opts=sq.Opts(2, 64, 64, 0)) == INVALID and "q_block" in _err()
    assert _fwd(opts=sq.Opts(8, 64, 64, 0)) == INVALID


def test_strided_forward_validation():
    L = sq.lib()
    good = (ctypes.c_int64 * 9)(*([3 * 2 * 64 * 64 * 8, 64, 3 * 2 * 64] * 3))
    bad = (ctypes.c_int64 * 9)(*([3 * 2 * 64 * 64 * 8, 64, 3 * 2 * 64 + 4] * 3))
    neg = (ctypes.c_int64 * 9)(*([-64, 64, 384] * 3))
    args = lambda st, ost=None: [FAKE, FAKE, FAKE, 1, 2, 64, 64, st, ost, 0.125, 0, None, FAKE, FAKE, 1, None, None]
    assert L.sqattn_forward_strided(*args(None)) == INVALID and "in_strides" in _err()
    assert L.sqattn_forward_strided(*args(bad)) == INVALID and "multiples of 8" in _err()
    assert L.sqattn_forward_strided(*args(neg)) == INVALID
    obad = (ctypes.c_int64 * 3)(8, 8, 12)
    assert L.sqattn_forward_strided(*args(good, obad)) == INVALID
    # valid strides reach the workspace check
    assert L.sqattn_forward_strided(*args(good)) == WORKSPACE


def test_rmsnorm_validation():
    L = sq.lib()
    args = lambda eps=1e-6, rows=10, cols=256, x=FAKE, inv=FAKE: [x, None, eps, rows, cols, FAKE, FAKE, inv, None]
    assert L.sqattn_w8a8_rmsnorm_quantize(*args(eps=0.0)) == INVALID and "eps" in _err()
    assert L.sqattn_w8a8_rmsnorm_quantize(*args(eps=float("nan"))) == INVALID
    assert L.sqattn_w8a8_rmsnorm_quantize(*args(cols=200)) == INVALID
    assert L.sqattn_w8a8_rmsnorm_quantize(*args(inv=None)) == INVALID and "inv_rms" in _err()
    assert L.sqattn_w8a8_rmsnorm_quantize(*args(rows=0, x=None, inv=None)) == OK
    assert L.sqattn_w8a8_rmsnorm_workspace_bytes(100, 256) > 100 * 256
    lin = [FAKE, None, 1e-6, FAKE, FAKE, None, 300, 200, 384, 0, FAKE, FAKE, 1, None]
    assert L.sqattn_w8a8_linear_rmsnorm(*lin) == WORKSPACE


def test_qknorm_forward_validation():
    L = sq.lib()
    H, N, d = 2, 64, 64
    fused = [3 * H * d * N, d, 3 * H * d]                 # [B, N, 3, H, d] views: head stride d
    good = (ctypes.c_int64 * 9)(*(fused * 3))
    bhnd = (ctypes.c_int64 * 9)(*([H * N * d, N * d, d] * 3))

    def call(st=good, eps=1e-6, gq=None, gk=None, H=H, wsb=1):
        return L.sqattn_forward_qknorm(FAKE, FAKE, FAKE, 1, H, N, d, st, None, gq, gk, eps, 0.125, 0, None, FAKE,
                                       FAKE, wsb, None, None)

    assert call(st=None) == INVALID and "in_strides" in _err()
    assert call(st=bhnd) == INVALID and "contiguous" in _err()
    assert call(eps=0.0) == INVALID and "eps" in _err()
    assert call(eps=float("inf")) == INVALID
    assert call(gq=FAKE + 2) == INVALID and "gamma_q" in _err()
    # valid arguments reach the workspace check, which counts the per-token factors
    assert call() == WORKSPACE
    plain = L.sqattn_workspace_bytes(1, H, N, d, 0, None)
    need = L.sqattn_forward_qknorm_workspace_bytes(1, H, N, d, 0, None)
    assert need >= plain + 2 * N * 4
    assert call(wsb=plain) == WORKSPACE
    # one head: any layout (the token's d values are a row)
    one = (ctypes.c_int64 * 9)(*([N * d, N * d, d] * 3))
    assert call(st=one, H=1) == WORKSPACE
    assert L.sqattn_forward_qknorm_workspace_bytes(1, H, N, 96, 0, None) == 0


def test_layernorm_validation():
    L = sq.lib()
    args = lambda eps=1e-6, rows=10, cols=256, x=FAKE, mean=FAKE, beta=None: [x, None, beta, eps, rows, cols, FAKE,
                                                                               FAKE, mean, FAKE, None]
    assert L.sqattn_w8a8_layernorm_quantize(*args(eps=-1.0)) == INVALID and "eps" in _err()
    assert L.sqattn_w8a8_layernorm_quantize(*args(cols=100)) == INVALID
    assert L.sqattn_w8a8_layernorm_quantize(*args(mean=None)) == INVALID and "mean" in _err()
    assert L.sqattn_w8a8_layernorm_quantize(*args(beta=FAKE + 1)) == INVALID and "beta" in _err()
    assert L.sqattn_w8a8_layernorm_quantize(*args(rows=0, x=None, mean=None)) == OK
    assert L.sqattn_w8a8_layernorm_workspace_bytes(100, 256) > L.sqattn_w8a8_rmsnorm_workspace_bytes(100, 256)
    lin = [FAKE, None, None, 1e-6, FAKE, FAKE, None, 300, 200, 384, 0, FAKE, FAKE, 1, None]
    assert L.sqattn_w8a8_linear_layernorm(*lin) == WORKSPACE
