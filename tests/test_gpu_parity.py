"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Quantization (INT8 codes, scales, K mean, E4M3 V codes and scales) must match
bit for bit over every row.  The attention output must agree within max-abs
1e-2 (plus the FP8 ambiguity envelope) and cosine >= 0.9999 over the checked
rows: every row for small cases, the seeded sample of 1024 rows per head
(which always holds the ragged last Q block) for the full-size workloads.
"""
import numpy as np
import pytest
import torch

import bit_quantized_attention_block_amd as sq
import workloads as W
from gpu_util import MAX_ABS, MIN_COS, check_fp8, dev_bf16, host, oracle_heads, out_metrics

pytestmark = pytest.mark.gpu


def _run_case(w, N=None, d=None, B=None, H=None, q_block=None, pv=None, heads=None, check_quant=True,
              data=None, per_row_scale=False, bound_hits=True):
    """per_row_scale: compare each output row divided by the largest |value|
    of the oracle's row (for inputs whose magnitude is far from 1);
    bound_hits: FP8 only, bound the fraction of ambiguous P elements (off for
    crafted extreme logits)."""
    pv = pv or w.pv
    q_block = q_block or w.q_block
    if data is None:
        q, k, v, rows = W.gen_inputs(w, N=N, d=d, B=B, H=H)
    else:
        q, k, v, rows = data
    B_, H_, N_, d_ = q.shape
    print(f"case {w.name} B={B_} H={H_} N={N_} d={d_} q_block={q_block} pv={pv}", flush=True)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    qi, qs, ki, ks, mu = sq.quantize_qk(Q, K, q_block, 64)
    out = sq.forward(Q, K, V, scale=w.scale, pv=pv, q_block=q_block)
    if pv == "fp8":
        vc, vs = sq.quantize_v_fp8(V)
    torch.cuda.synchronize()
    ref = oracle_heads(q, k, v, rows, q_block, w.scale, pv, heads=heads)
    idx = [i for i in range(B_ * H_) if ref[i] is not None]
    if check_quant:
        qi_h, qs_h, ki_h, ks_h, mu_h = (host(x) for x in (qi, qs, ki, ks, mu))
        for i in idx:
            b, h = divmod(i, H_)
            r = ref[i]
            assert np.array_equal(mu_h[b, h].view(np.uint32), r["k_mean"].view(np.uint32)), f"k_mean head {i}"
            assert np.array_equal(qs_h[b, h].view(np.uint32), r["q_scale"].view(np.uint32)), f"q_scale head {i}"
            assert np.array_equal(ks_h[b, h].view(np.uint32), r["k_scale"].view(np.uint32)), f"k_scale head {i}"
            assert np.array_equal(qi_h[b, h], r["q_codes"]), f"q codes head {i}"
            assert np.array_equal(ki_h[b, h], r["k_codes"]), f"k codes head {i}"
        if pv == "fp8":
            vc_h, vs_h = host(vc), host(vs)
            for i in idx:
                b, h = divmod(i, H_)
                assert np.array_equal(vs_h[b, h].view(np.uint32), ref[i]["v_scale"].view(np.uint32))
                assert np.array_equal(vc_h[b, h], ref[i]["v_codes"]), f"v codes head {i}"
    out_h = host(out)
    g_rows, r_rows, e_rows = [], [], []
    for i in idx:
        b, h = divmod(i, H_)
        g, r, e = out_h[b, h][rows[i]], ref[i]["out"], ref[i]["envelope"]
        if per_row_scale:
            sc = np.maximum(np.abs(r).max(axis=1, keepdims=True), np.finfo(np.float64).tiny)
            g, r, e = g / sc, r / sc, (None if e is None else e / sc)
        g_rows.append(g)
        r_rows.append(r)
        e_rows.append(e)
    m = out_metrics(g_rows, r_rows, e_rows if pv == "fp8" else None)
    print(f"  max_abs={m['max_abs']:.3e} excess={m['max_excess']:.3e} env={m['env_max']:.2e} "
          f"cos={m['cos']:.8f}", flush=True)
    assert np.isfinite(out_h).all()
    assert m["max_excess"] <= MAX_ABS, m
    assert m["cos"] >= MIN_COS, m
    if pv == "fp8":
        check_fp8(m, sum(ref[i]["envelope_hits"] for i in idx), sum(len(rows[i]) * N_ for i in idx),
                  bound_hits=bound_hits)
    return m


def test_tiny_workload_all_rows():
    _run_case(W.get(0))


def test_tiny_workload_fp8():
    _run_case(W.get(0), pv="fp8")


@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 129, 255, 257, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths_bf16(N, d):
    _run_case(W.get(1), N=N, d=d, B=1, H=2)


@pytest.mark.parametrize("N", [1, 63, 65, 129, 300, 777])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths_fp8(N, d):
    _run_case(W.get(3), N=N, d=d, B=1, H=2)


@pytest.mark.parametrize("q_block", [16, 64, 192, 256])
def test_q_block_sizes(q_block):
    _run_case(W.get(1), N=700, d=128, B=2, H=3, q_block=q_block)


def test_several_work_groups_and_heads():
    # many query tiles and many heads: the XCD-ordered work list must cover all
    _run_case(W.get(2), N=2000, d=128, B=2, H=9)


def _degenerate(kind, N=333, d=128):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, N, d))
    k = rng.standard_normal((1, 2, N, d)) + 2.0
    v = rng.standard_normal((1, 2, N, d))
    if kind == "zero_q":
        q[:] = 0.0
    elif kind == "constant_k":          # K' = 0 everywhere: all K scales 0, uniform attention
        k[:] = np.linspace(-1, 1, d)[None, None, None, :]
    elif kind == "constant_v":
        v[:] = np.linspace(-3, 3, d)[None, None, None, :]
    elif kind == "zero_v_block":
        v[:, :, 64:128] = 0.0
    elif kind == "one_hot":             # one key aligned with every query dominates
        q[:] = 1.0
        k[:, :, 100] = 6.0
    elif kind == "far_max":             # that key's score exceeds the first keys' by far more
        q[:] = 1.0                      # than the fp32 range: the exact-max recomputation
        k[:, :, 100] = 20.0
    elif kind == "v_scale_spread":      # V blocks 2^-40 .. 2^40 apart: per-block FP8 scales
        e = rng.integers(-40, 41, size=(N + 63) // 64)  # that differ by up to 2^80
        v *= np.exp2(np.repeat(e, 64)[:N])[None, None, :, None]
    cvt = lambda x: W.f32_to_bf16_bits(x.astype(np.float32))
    rows = [np.arange(N)] * 2
    return cvt(q), cvt(k), cvt(v), rows


@pytest.mark.parametrize("kind", ["zero_q", "constant_k", "constant_v", "zero_v_block", "one_hot", "far_max",
                                  "v_scale_spread"])
@pytest.mark.parametrize("pv", ["bf16", "fp8"])
def test_degenerate_inputs(kind, pv):
    _run_case(W.get(1), pv=pv, q_block=128, data=_degenerate(kind), per_row_scale=kind == "v_scale_spread",
              bound_hits=False)


def test_second_pass_counter():
    # opts.second_pass_count counts the work items (head, 256-row block) that
    # took the exact-max second pass.  far_max: every row's score at key 100
    # exceeds its first 32 keys' by about 290 in log2 units, so every one of
    # the 2 heads x 2 blocks does; workload-shaped data never does.  The
    # counter leaves the output unchanged and accumulates over calls.
    q, k, v, _ = _degenerate("far_max")
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = sq.forward(Q, K, V, pv="bf16")
    out = sq.forward(Q, K, V, pv="bf16", second_pass_count=cnt)
    out = sq.forward(Q, K, V, pv="bf16", second_pass_count=cnt, out=out)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 2 * 4 and torch.equal(out, ref)
    qi, qs, ki, ks, _ = sq.quantize_qk(Q, K, 128, 64)
    cnt.zero_()
    sq.attend_quantized(qi, qs, ki, ks, V, pv="bf16", second_pass_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 4
    w = W.get(2)
    q, k, v, _ = W.gen_inputs(w, N=1500, d=128, B=1, H=3)
    cnt.zero_()
    for pv in ("bf16", "fp8"):
        sq.forward(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=w.scale, pv=pv, second_pass_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0


def test_attend_quantized_matches_forward():
    # sqattn_attend_quantized (raw V or E4M3 codes) and sqattn_attend_packed
    # (V in the kernel's tile layout) give the forward's bytes
    w = W.get(2)
    q, k, v, rows = W.gen_inputs(w, N=1500, d=128, B=1, H=3)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for pv in ("bf16", "fp8"):
        out = sq.forward(Q, K, V, scale=w.scale, pv=pv)
        qi, qs, ki, ks, mu = sq.quantize_qk(Q, K, 128, 64)
        if pv == "fp8":
            vc, vs = sq.quantize_v_fp8(V)
            out2 = sq.attend_quantized(qi, qs, ki, ks, vc, vs, scale=w.scale, pv=pv)
            out3 = sq.attend_packed(qi, qs, ki, ks, sq.pack_v(vc, pv), vs, scale=w.scale, pv=pv)
        else:
            out2 = sq.attend_quantized(qi, qs, ki, ks, V, scale=w.scale, pv=pv)
            out3 = sq.attend_packed(qi, qs, ki, ks, sq.pack_v(V, pv), scale=w.scale, pv=pv)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(out, out3), pv


@pytest.mark.parametrize("pv", ["bf16", "fp8"])
def test_plain_forward_entry_point(pv):
    # sqattn_forward(q, k, v, B, H, N, d, scale, pv_dtype, out, ...) called through
    # the C symbol itself (default blocks: q 128, k/v 64; fp32 out): every row of
    # a ragged 300-token case against the oracle, and equal to sqattn_forward_ex
    import ctypes
    w = W.get(0)
    q, k, v, rows = W.gen_inputs(w, N=300, d=64, B=1, H=2)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    B, H, N, d = q.shape
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    L = sq.lib()
    st = torch.cuda.current_stream().cuda_stream
    code = {"bf16": sq.PV_BF16, "fp8": sq.PV_FP8}[pv]
    rc = L.sqattn_forward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), B, H, N, d, ctypes.c_float(w.scale), code,
                          out.data_ptr(), None, 0, st)
    assert rc == 0, sq.lib().sqattn_last_error()
    ex = torch.empty_like(out)
    rc = L.sqattn_forward_ex(Q.data_ptr(), K.data_ptr(), V.data_ptr(), B, H, N, d, ctypes.c_float(w.scale), code,
                             ex.data_ptr(), None, 0, st, None)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ex)
    ref = oracle_heads(q, k, v, rows, 128, w.scale, pv)
    got = host(out)
    m = out_metrics([got[0, i][rows[i]] for i in range(H)], [ref[i]["out"] for i in range(H)],
                    [ref[i]["envelope"] for i in range(H)] if pv == "fp8" else None)
    assert m["max_abs"] <= MAX_ABS and m["cos"] >= MIN_COS, m


def test_k_out_of_accumulator_range_gives_nan_mean():
    # a head holding |K| >= 2^33 is outside the exact K-mean accumulator: its
    # mean is NaN (a finite value elsewhere in the batch is unaffected)
    w = W.get(0)
    q, k, v, rows = W.gen_inputs(w, N=200, d=64, B=1, H=2)
    k = k.copy()
    k[0, 0, 17, 5] = W.f32_to_bf16_bits(np.array([2.0 ** 34], np.float32))[0]
    Q, K = dev_bf16(q), dev_bf16(k)
    qi, qs, ki, ks, mu = sq.quantize_qk(Q, K, 64, 64)
    torch.cuda.synchronize()
    mu_h, ks_h, ki_h = host(mu), host(ks), host(ki)
    assert np.isnan(mu_h[0, 0]).all()
    ref = oracle_heads(q, k, v, rows, 64, w.scale, "bf16", heads=[1])[1]
    assert np.array_equal(mu_h[0, 1].view(np.uint32), ref["k_mean"].view(np.uint32))
    assert np.array_equal(ks_h[0, 1].view(np.uint32), ref["k_scale"].view(np.uint32))
    assert np.array_equal(ki_h[0, 1], ref["k_codes"])


def test_deterministic_and_caller_workspace():
    w = W.get(1)
    q, k, v, rows = W.gen_inputs(w, N=5000, d=128, B=1, H=4)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for pv in ("bf16", "fp8"):
        a = sq.forward(Q, K, V, pv=pv)
        nb = sq.workspace_bytes(1, 4, 5000, 128, pv)
        ws = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")   # dirty workspace
        b = sq.forward(Q, K, V, pv=pv, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b), pv


@pytest.mark.parametrize("pv", ["bf16", "fp8"])
def test_deterministic_full_grid(pv):
    """A full Wan-14B-480p-sized grid (1x40x32760x128) twice: identical bits.
    Under a full grid the tile loads stay in flight across tile boundaries, so
    a read that races its load shows up here as run-to-run differences."""
    g = torch.Generator(device="cuda").manual_seed(11)
    shape = (1, 40, 32760, 128)
    Q, K, V = (torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    outs = [sq.forward(Q, K, V, pv=pv) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0], o), pv
    assert bool(torch.isfinite(outs[0]).all())


@pytest.mark.parametrize("pv", ["bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_output(pv, d):
    """opts.out_dtype = bf16: the fp32 result rounded to nearest even, bit for
    bit, from both entry points; and within the parity bound plus one bf16
    ulp of the oracle."""
    w = W.get(1)
    q, k, v, rows = W.gen_inputs(w, N=700, d=d, B=1, H=2)
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o32 = sq.forward(Q, K, V, scale=w.scale, pv=pv)
    o16 = sq.forward(Q, K, V, scale=w.scale, pv=pv, out_dtype=torch.bfloat16)
    qi, qs, ki, ks, mu = sq.quantize_qk(Q, K, w.q_block, 64)
    if pv == "fp8":
        vc, vs = sq.quantize_v_fp8(V)
        a16 = sq.attend_quantized(qi, qs, ki, ks, vc, vs, scale=w.scale, pv=pv, out=torch.empty_like(o16))
    else:
        a16 = sq.attend_quantized(qi, qs, ki, ks, V, scale=w.scale, pv=pv, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16 and a16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(a16, o16)
    ref = oracle_heads(q, k, v, rows, w.q_block, w.scale, pv)
    got = host(o16.float())
    for i in range(2):
        r = ref[i]["out"]
        e = ref[i]["envelope"] if pv == "fp8" else 0.0
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
        assert (np.abs(got[0, i][rows[i]] - r) <= MAX_ABS + e + ulp).all()


def test_workspace_too_small_raises():
    Q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(sq.SqattnError, match="workspace"):
        sq.forward(Q, Q, Q, workspace=ws)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("pv", ["bf16", "fp8"])
def test_long_sequence(pv):
    """One head of 2^19 + 37 tokens (d = 64): 8193 key tiles with a ragged
    last Q block and K tile.  Checked rows: the whole last Q block plus 200
    seeded ones."""
    w = W.get(3 if pv == "fp8" else 2)
    N = (1 << 19) + 37
    q, k, v, _ = W.gen_inputs(w, N=N, d=64, B=1, H=1)
    rng = np.random.default_rng(20)
    tail = np.arange(N - N % w.q_block, N)
    rows = [np.concatenate([np.sort(rng.choice(N - len(tail), 200, replace=False)), tail])]
    _run_case(w, pv=pv, data=(q, k, v, rows))


@pytest.mark.timeout(900)
def test_offsets_past_2gib():
    """140 heads of 32760 x 128: the fp32 output spans 2.35e9 bytes, so the
    last head's rows sit past 2^31 bytes (and its Q/K/V past 2^30); that head
    is checked against the oracle on 256 seeded rows (with its ragged tail)."""
    w = W.get(2)
    H = 140
    q, k, v, rows = W.gen_inputs(w, H=H)
    assert q.size * 4 > (1 << 31)
    rows = [r[-256:] for r in rows]
    _run_case(w, data=(q, k, v, rows), heads=[H - 1])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_full_size_workload(index):
    """The Wan-shaped workloads at full size: quantization bit-exact on every
    row of every head, output on 1024 seeded rows per head."""
    _run_case(W.get(index))


@pytest.mark.parametrize("pv,d", [("bf16", 128), ("bf16", 64), ("fp8", 128), ("fp8", 64)])
def test_per_row_q_scales(pv, d):
    """q_block = 1: one Q scale per row (the Q operand's per-lane granularity);
    the bf16 path on the normal workloads, the FP8 path on the heavy-tailed
    one, as the workload table pairs them."""
    _run_case(W.get(1 if pv == "bf16" else 3), N=777, d=d, B=1, H=3, q_block=1, pv=pv)


@pytest.mark.timeout(900)
def test_per_row_q_scales_full_size_heavy_tailed():
    """The heavy-tailed FP8 workload with per-row Q scales, every 8th head."""
    _run_case(W.get(3), q_block=1, heads=range(0, 40, 8))
