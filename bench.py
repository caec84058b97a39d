#!/usr/bin/env python3
"""Throughput of the quantized-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

With a W8A8 workload (--workload w8a8-qkv-wan14b-480p and the other w8a8-*
names) it measures the block-wise INT8 linear layer instead; see bench_w8a8.
With --block-density D it measures block-sparse attention: a seeded mask
(local band plus a fraction D of the other 128-row x 64-key blocks) and TOPS
over the kept blocks' work only; see sparse_ops.

One step is one full sqattn_forward over the workload: exact K mean, INT8
quantization of Q and smoothed K, V packing (or E4M3 quantization), and the
attention kernel, from bf16 Q/K/V resident in HBM to the fp32 output in HBM.
The metric is TOPS = 4*B*H*N^2*d / time, also reported as a percentage of the
MI355X dense INT8 matrix peak (5.0 POPS).

Printed: one JSON line with the contract fields plus
  roofline     - the attention kernel alone (its average launch duration from
                 HIP events on the launch stream), against the INT8 MFMA peak
                 (`frac`) and against the mixed ceiling of its two products
                 (`frac_mixed`: Q K^T on INT8 at 5.0 POPS, P V on bf16 at 2.5
                 or on FP8 at 5.0 PFLOP/s); `traffic` comes from the rocprofv3
                 counter summary in profiles/ when it was taken on the current
                 kernel source and headers;
  cpu_baseline - the CPU oracle timed on a bounded sample of the same workload
                 (ten heads), scaled to the whole workload;
  numerics     - the error of the GPU output on that sample's rows against the
                 oracle and against unquantized float64 attention;
  fallback     - how many work items took the 16-bit path's exact-max second
                 pass (opts.second_pass_count) in one forward;
  system       - GPU, ROCm, hipcc, driver and torch versions and the shader and
                 memory clocks sampled while the timed steps ran.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0        # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0         # dense FP8 MFMA
METRIC = "quantized-attention TOPS (4·B·H·N²·d/s) + % of MI355X INT8 MFMA peak"
W8A8_METRIC = "W8A8 linear INT8 TOPS (2·M·N·K/s) + % of MI355X INT8 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic.json")
CSRC = os.path.join(ROOT, "bit_quantized_attention_block_amd", "csrc")
# the attention kernel source of each P.V path
ATTN_SRC = {"bf16": os.path.join(CSRC, "attn_bf16.hip"), "fp8": os.path.join(CSRC, "attn_fp8.hip")}
ATTN_KERNEL = {"bf16": "attn_bf16_kernel", "fp8": "attn_fp8_kernel"}
W8A8_SRC = os.path.join(CSRC, "w8a8.hip")
W8A8_KERNEL = "w8a8_gemm_kernel"


def _profiled(name, src):
    """The committed counter summary of the workload's profiled kernel, or
    None if absent or taken on another version of the kernel source or of a
    header it includes."""
    from bit_quantized_attention_block_amd.rocprof_harness import source_key
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(name)
    except (OSError, ValueError, AttributeError):
        return None
    if not t or t.get("src_key") != source_key(src):
        return None
    return t


def _traffic(name, src):
    """Per-launch HBM bytes of the workload's profiled kernel (see _profiled)."""
    t = _profiled(name, src)
    return t.get("bytes_per_launch") if t else None


def _at_profiled_clock(roof, name, src):
    """Adds the sustained shader clock of the profiled run (GRBM cycles per
    XCD over the kernel time) and the roofline fractions against the peaks
    scaled to that clock (the quoted peaks assume 2.4 GHz)."""
    t = _profiled(name, src)
    clk = t.get("sustained_clock_ghz") if t else None
    roof["profiled_clock_ghz"] = round(clk, 4) if clk else None
    roof["frac_at_profiled_clock"] = round(roof["frac"] * 2.4 / clk, 4) if clk else None
    roof["frac_mixed_at_profiled_clock"] = round(roof["frac_mixed"] * 2.4 / clk, 4) if clk else None
    # matrix-core utilisation of the profiled run: its counted MFMA ops per
    # operand type over what the matrix cores do in its cycles
    mu = t.get("mfma_utilisation") if t else None
    roof["mfma_utilisation_profiled"] = round(mu, 4) if mu else None
    return roof


def mixed_peak(pv):
    """The MFMA ceiling of attention in ops/s units (TOPS): half the work
    (Q K^T) on INT8 at 5.0 POPS, half (P V) on bf16 at 2.5 or FP8 at 5.0
    PFLOP/s, so 4 / (2/5.0 + 2/peak_pv) POPS."""
    pv_peak = BF16_PEAK_TFLOPS if pv == "bf16" else FP8_PEAK_TFLOPS
    return 1.0 / (0.5 / INT8_PEAK_TOPS + 0.5 / pv_peak)


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def _cmd(*args):
    try:
        r = subprocess.run(list(args), capture_output=True, text=True, timeout=20)
        return r.stdout if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def _card(torch):
    """sysfs device directory of cuda:0 (matched by PCI bus id when several
    cards are listed), or None."""
    import glob
    cards = sorted(c for c in glob.glob("/sys/class/drm/card[0-9]*/device") if os.path.exists(c + "/pp_dpm_sclk"))
    if len(cards) == 1:
        return cards[0]
    try:
        p = torch.cuda.get_device_properties(0)
        bus = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}"
    except Exception:
        return None
    for c in cards:
        if bus in os.path.realpath(c):
            return c
    return None


def _dpm_mhz(text):
    """The current level (marked '*') of a pp_dpm_* listing, in MHz."""
    for line in (text or "").splitlines():
        if line.rstrip().endswith("*"):
            v = line.split(":", 1)[-1].strip().rstrip("*").strip().lower()
            try:
                return float(v.replace("mhz", ""))
            except ValueError:
                return None
    return None


class ClockSampler:
    """Samples the current shader and memory clock levels from sysfs every
    interval seconds on a thread while the timed steps run."""

    def __init__(self, card, interval=0.02):
        self.card, self.interval = card, interval
        self.sclk, self.mclk = [], []
        self._stop = threading.Event()
        self._t = None

    def __enter__(self):
        if self.card:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            s = _dpm_mhz(_read(self.card + "/pp_dpm_sclk"))
            m = _dpm_mhz(_read(self.card + "/pp_dpm_mclk"))
            if s:
                self.sclk.append(s)
            if m:
                self.mclk.append(m)
            self._stop.wait(self.interval)

    def __exit__(self, *exc):
        self._stop.set()
        if self._t:
            self._t.join()

    def summary(self):
        import numpy as np
        if not self.sclk:
            return {"source": "sysfs pp_dpm_sclk / pp_dpm_mclk", "samples": 0,
                    "note": "not readable on this machine" if self.card is None else "no samples"}
        s = np.array(self.sclk)
        return {"source": f"sysfs pp_dpm_sclk / pp_dpm_mclk current level every {self.interval * 1e3:.0f} ms "
                          "during the timed forward steps",
                "samples": int(s.size), "sclk_mhz_median": float(np.median(s)), "sclk_mhz_min": float(s.min()),
                "sclk_mhz_max": float(s.max()),
                "mclk_mhz_median": float(np.median(self.mclk)) if self.mclk else None}


def system_info(torch):
    """GPU name and architecture, ROCm / HIP runtime / hipcc / driver / torch
    versions."""
    info = {"torch": torch.__version__, "hip_runtime": torch.version.hip,
            "rocm": _read("/opt/rocm/.info/version"),
            "driver": _read("/sys/module/amdgpu/version")}
    try:
        p = torch.cuda.get_device_properties(0)
        info["gpu"] = p.name
        info["arch"] = getattr(p, "gcnArchName", None)
        info["compute_units"] = p.multi_processor_count
    except Exception:  # pragma: no cover
        pass
    hv = _cmd("/opt/rocm/bin/hipcc", "--version") or ""
    info["hipcc"] = "; ".join(l.strip() for l in hv.splitlines() if "version" in l.lower())[:200] or None
    if not info["driver"]:
        dv = _cmd("/opt/rocm/bin/rocm-smi", "--showdriverversion") or ""
        info["driver"] = next((l.split(":", 1)[-1].strip() for l in dv.splitlines()
                               if "driver version" in l.lower() and ":" in l), None)
    return info


def _timed(torch, np, dev, stream, fn, n):
    """Average, median and minimum ms of n calls of fn, from HIP events on the
    launch stream (one event after every call), and the wall time of the n
    calls (launch to completion)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize(dev)
    wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    return ev[0].elapsed_time(ev[n]) / n, float(np.median(per)), min(per), wall


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def _cores():
    """(CPU cores this process may run on, BLAS threads of numpy)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        n = os.cpu_count() or 1
    return n, _blas_threads()


def cpu_baseline_w8a8(w, x, wt, b, row_blocks=64, w_rows=8192):
    """Time the oracle on a sample of the layer: INT8 quantization of
    `row_blocks` 128-row blocks of x and the block-scaled product of those rows
    with the first `w_rows` rows of W (quantized by the oracle too, untimed:
    the weights are quantized once, off the step), scaled to the whole layer."""
    import numpy as np
    import oracle
    import workloads as W
    rows = min(w.M, 128 * row_blocks)
    wr = min(w.N, w_rows)
    cw, sw = oracle.w8a8.quantize_blocks(W.bf16_bits_to_f32(wt[:wr]))
    t0 = time.perf_counter()
    cx, sx = oracle.w8a8.quantize_blocks(W.bf16_bits_to_f32(x[:rows]))
    t1 = time.perf_counter()
    oracle.w8a8.linear(cx, sx, cw, sw, None if b is None else b[:wr])
    t2 = time.perf_counter()
    t_full = (t1 - t0) / rows * w.M + (t2 - t1) / (rows * wr) * (w.M * w.N)
    cores, blas = _cores()
    return {"value": round(w.ops / t_full / 1e12, 6), "unit": "TOPS", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"{rows} rows of x quantized ({t1 - t0:.1f} s) and multiplied with {wr} of the {w.N} rows "
                      f"of W ({t2 - t1:.1f} s); scaled to {w.M} x {w.N} outputs",
            "sample_seconds": round(t2 - t0, 2)}


def numerics_w8a8(w, x, wt, b, y_dev, rows=1024, cols=1024):
    """Error of the GPU layer output (bf16) on the first rows x cols outputs:
    against the oracle, also as a ratio to the rounding bound of the kernel's
    fp32 evaluation ((n + 2) 2^-24 sum_j |sx sw D_j|, n slices) plus a bf16
    step of the result, and against the unquantized float64 product of the
    same bf16 inputs (the method's own error).  Whole 128-row blocks, so the
    sample's scales are the layer's."""
    import numpy as np

    import oracle
    import workloads as W
    r, c = min(w.M, rows), min(w.N, cols)
    xf, wf = W.bf16_bits_to_f32(x[:r]), W.bf16_bits_to_f32(wt[:c])
    cx, sx = oracle.w8a8.quantize_blocks(xf)
    cw, sw = oracle.w8a8.quantize_blocks(wf)
    bb = None if b is None else np.asarray(b[:c], np.float32)
    ref = oracle.w8a8.linear(cx, sx, cw, sw, bb)
    tol = (w.K // 128 + 2) * 2.0 ** -24 * oracle.w8a8.linear_bound(cx, sx, cw, sw, bb) + 2.0 ** -8 * np.abs(ref)
    g = y_dev[:r, :c].float().cpu().numpy().astype(np.float64)
    e = np.abs(g - ref)
    exact = xf.astype(np.float64) @ wf.astype(np.float64).T
    if bb is not None:
        exact += bb.astype(np.float64)[None, :]
    dq = np.abs(g - exact)
    return {"outputs": f"rows 0..{r - 1} x columns 0..{c - 1}",
            "vs_oracle_max_abs": float(e.max()),
            "vs_oracle_max_over_bound": float((e / np.maximum(tol, 1e-300)).max()),
            "vs_fp64_unquantized_max_abs": float(dq.max()),
            "vs_fp64_unquantized_mean_abs": float(dq.mean()),
            "vs_fp64_unquantized_rel_rms": float(np.sqrt((dq ** 2).mean() / (exact ** 2).mean()))}


def bench_w8a8(a):
    """One step = the W8A8 layer on bf16 activations in HBM: INT8 quantization
    of x (128x128 blocks) and the block-scaled INT8 GEMM with bias, bf16
    output; the weights are quantized once before timing, as a deployed
    model stores them.  TOPS = 2*M*N*K / time."""
    import numpy as np
    import torch

    import bit_quantized_attention_block_amd as sq
    from workloads import linear as WL

    w = WL.get_linear(a.workload)
    t0 = time.perf_counter()
    x, wt, b = WL.gen_x(w), WL.gen_w(w), WL.gen_bias(w)
    print(f"[bench] generated {w.name} inputs in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    to = lambda v: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
    X = to(x)
    wc, ws = sq.w8a8_quantize(to(wt))
    B = torch.from_numpy(b).to(dev) if b is not None else None
    Y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    wsb = torch.empty(sq.w8a8_workspace_bytes(w.M, w.K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    G = torch.ones(w.K, dtype=torch.float32, device=dev) * 1.25
    Be = torch.full((w.K,), 0.1, dtype=torch.float32, device=dev)
    if a.rmsnorm:
        wsb = torch.empty(sq.w8a8_rmsnorm_workspace_bytes(w.M, w.K), dtype=torch.uint8, device=dev)
    if a.layernorm:
        wsb = torch.empty(sq.w8a8_layernorm_workspace_bytes(w.M, w.K), dtype=torch.uint8, device=dev)

    def step():
        if a.rmsnorm:
            sq.w8a8_linear_rmsnorm(X, wc, ws, gamma=G, eps=1e-6, bias=B, out=Y, workspace=wsb)
        elif a.layernorm:
            sq.w8a8_linear_layernorm(X, wc, ws, gamma=G, beta=Be, eps=1e-6, bias=B, out=Y, workspace=wsb)
        else:
            sq.w8a8_linear(X, wc, ws, bias=B, out=Y, workspace=wsb)

    for _ in range(a.warmup):
        step()
    with ClockSampler(_card(torch)) as clocks:
        ms, ms_med, ms_min, t_wall = _timed(torch, np, dev, stream, step, a.steps)
    print(f"[bench] linear {ms:.3f} ms/step (median {ms_med:.3f}, min {ms_min:.3f}; wall "
          f"{t_wall / a.steps * 1e3:.3f}); torch {torch.__version__}, HIP {torch.version.hip}",
          file=sys.stderr, flush=True)
    xc, xs = sq.w8a8_quantize(X)

    def kern():
        sq.w8a8_gemm(xc, xs, wc, ws, bias=B, out=Y)

    reps = a.kernel_reps or a.steps
    for _ in range(2):
        kern()
    k_ms, k_med, k_min, _ = _timed(torch, np, dev, stream, kern, reps)
    ops = w.ops
    q_ms = _timed(torch, np, dev, stream, lambda: sq.w8a8_quantize(X), reps)[0]
    n_ms = _timed(torch, np, dev, stream, lambda: sq.w8a8_rmsnorm_quantize(X, G, 1e-6), reps)[0]
    l_ms = _timed(torch, np, dev, stream, lambda: sq.w8a8_layernorm_quantize(X, G, Be, 1e-6), reps)[0]
    tops = ops / (ms * 1e-3) / 1e12
    k_tops = ops / (k_ms * 1e-3) / 1e12
    res = {
        "metric": W8A8_METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "pct_int8_peak": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "block": 128, "bias": b is not None,
                   "out": "bf16",
                   "stages_ms": {"step_median": round(ms_med, 4), "step_min": round(ms_min, 4),
                                 "gemm_kernel": round(k_ms, 4), "gemm_kernel_median": round(k_med, 4),
                                 "gemm_kernel_min": round(k_min, 4), "quantize_x": round(q_ms, 4),
                                 "rmsnorm_quantize_x": round(n_ms, 4), "layernorm_quantize_x": round(l_ms, 4)},
                   "rmsnorm": bool(a.rmsnorm), "layernorm": bool(a.layernorm)},
        "roofline": _at_profiled_clock(
            {"kernel": W8A8_KERNEL, "bound": "mfma", "achieved": round(k_tops, 2),
             "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(k_tops / INT8_PEAK_TOPS, 4),
             "peak_mixed": INT8_PEAK_TOPS, "frac_mixed": round(k_tops / INT8_PEAK_TOPS, 4),
             "traffic": _traffic(w.name, W8A8_SRC), "avg_launch_ms": round(k_ms, 4),
             "ops_per_launch": w.ops}, w.name, W8A8_SRC),
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_w8a8(w, x, wt, b)
        # Y holds the plain layer's output of the last kernel launches
        res["numerics"] = numerics_w8a8(w, x, wt, b, Y)
    else:
        res["cpu_baseline"] = None
        res["numerics"] = None
    res["system"] = system_info(torch)
    res["system"]["clocks"] = clocks.summary()
    print(json.dumps(res), flush=True)
    return 0


def sparse_ops(w, mask):
    """(kept, processed) operation counts of block-sparse attention: kept =
    4 d x the (query row, key) pairs of the kept blocks; processed = what the
    kernel computes, each 256-row work-group running the union of its two
    mask rows' tiles over all its rows."""
    import numpy as np
    N, d = w.N, w.d
    mq, nt = mask.shape[2], mask.shape[3]
    rows = np.minimum(128, N - 128 * np.arange(mq)).astype(np.float64)
    keys = np.minimum(64, N - 64 * np.arange(nt)).astype(np.float64)
    kept = 4.0 * d * np.einsum("bhij,i,j->", mask.astype(np.float64), rows, keys)
    m = mask.astype(bool)
    if mq % 2:
        m = np.concatenate([m, np.zeros(m.shape[:2] + (1, nt), bool)], axis=2)
    union = m[:, :, 0::2] | m[:, :, 1::2]
    wrows = np.minimum(256, N - 256 * np.arange(union.shape[2])).astype(np.float64)
    processed = 4.0 * d * np.einsum("bhij,i,j->", union.astype(np.float64), wrows, keys)
    return int(kept), int(processed)


def cpu_baseline(w, q, k, v, rows, heads=10, mask=None, ops=None, outs=None):
    """Time the oracle on `heads` heads (full quantization of each head plus
    its checked rows against all N keys) and scale to the whole workload
    (with a block mask: the masked oracle, rated on the kept work `ops`).
    The oracle's output rows go into `outs` ({(b, h): (rows, O, E)}, E the
    FP8 path's per-element ambiguity bound, else None)."""
    import numpy as np
    import oracle
    cores, blas = _cores()
    t_quant = t_attn = 0.0
    nrows = 0
    for i in range(heads):
        b, h = divmod(i, w.H)
        t0 = time.perf_counter()
        qc, qs = oracle.quant.quantize_q(q[b, h], w.q_block)
        kc, ks, mu = oracle.quant.quantize_k(k[b, h], w.k_block)
        if w.pv == "fp8":
            vc, vs = oracle.quant.quantize_v_fp8(v[b, h], 64)
        t1 = time.perf_counter()
        r = rows[i]
        bm = None if mask is None else mask[b, h]
        if w.pv == "fp8":
            O, E, _ = oracle.attention.attend_fp8(qc, qs, kc, ks, vc, vs, r, w.q_block, w.k_block, w.scale,
                                                  block_mask=bm)
        else:
            O = oracle.attention.attend_bf16(qc, qs, kc, ks, v[b, h], r, w.q_block, w.k_block, w.scale,
                                             block_mask=bm)
            E = None
        t2 = time.perf_counter()
        if outs is not None:
            outs[(b, h)] = (r, O, E)
        t_quant += t1 - t0
        t_attn += t2 - t1
        nrows += len(r)
    BH = w.B * w.H
    t_full = t_quant / heads * BH + t_attn / nrows * (w.N * BH)
    return {"value": round((w.ops if ops is None else ops) / t_full / 1e12, 6), "unit": "TOPS",
            "cores": cores, "blas_threads": blas, "kind": "oracle",
            "sample": f"{heads} heads of {w.name}: full quantization ({t_quant:.1f} s) + {nrows} query rows "
                      f"against all {w.N} keys ({t_attn:.1f} s); scaled to {BH} heads x {w.N} rows"
                      + ("" if mask is None else " (block mask applied)"),
            "sample_seconds": round(t_quant + t_attn, 2),
            # query rows per second: of the whole job (quantization included,
            # as scaled above) and of the attention alone on the sample
            "rows_per_s": round(w.N * BH / t_full, 3),
            "attention_rows_per_s": round(nrows / t_attn, 3)}


def numerics(w, q, k, v, out, outs, mask=None):
    """Error of the GPU output on the oracle's sampled rows: against the
    oracle (the parity measure; for FP8 also beyond its per-element ambiguity
    bound) and against unquantized float64 attention on the same bf16 inputs
    (the method's own error)."""
    import numpy as np
    import torch

    import oracle
    import workloads as W
    worst = dict(oracle_max_abs=0.0, oracle_max_excess=0.0, fp64_max_abs=0.0, fp64_mean_abs=0.0)
    cos_min, n, s_abs = 1.0, 0, 0.0
    for (b, h), (r, O, E) in outs.items():
        g = out[b, h][torch.as_tensor(r, device=out.device)].float().cpu().numpy().astype(np.float64)
        e = np.abs(g - O)
        worst["oracle_max_abs"] = max(worst["oracle_max_abs"], float(e.max()))
        if E is not None:
            worst["oracle_max_excess"] = max(worst["oracle_max_excess"], float(np.maximum(e - E, 0).max()))
        if mask is not None:
            continue
        f = W.bf16_bits_to_f32
        ref = oracle.attention.attention_fp64(f(q[b, h, r]).astype(np.float64), f(k[b, h]).astype(np.float64),
                                              f(v[b, h]).astype(np.float64), w.scale)
        d = np.abs(g - ref)
        worst["fp64_max_abs"] = max(worst["fp64_max_abs"], float(d.max()))
        s_abs += float(d.sum())
        n += d.size
        cos = (g * ref).sum(1) / np.maximum(np.linalg.norm(g, axis=1) * np.linalg.norm(ref, axis=1), 1e-300)
        cos_min = min(cos_min, float(cos.min()))
    res = {"rows": int(sum(len(r) for r, _, _ in outs.values())),
           "vs_oracle_max_abs": worst["oracle_max_abs"]}
    if w.pv == "fp8":
        res["vs_oracle_max_abs_beyond_fp8_ambiguity"] = worst["oracle_max_excess"]
    if mask is None:
        res.update({"vs_fp64_unquantized_max_abs": worst["fp64_max_abs"],
                    "vs_fp64_unquantized_mean_abs": s_abs / max(n, 1), "vs_fp64_unquantized_cos_min": cos_min})
    return res


def bench_dit_block(a):
    """The DiT attention block of the Wan-14B-480p shape from the library's
    fused pieces: LayerNorm (modulation as gamma, beta) fused into the W8A8
    QKV projection, attention with the q/k RMSNorm fused on views of its
    output, the W8A8 output projection on the attention output in place."""
    import numpy as np
    import torch

    import bit_quantized_attention_block_amd as sq
    import workloads as W

    w = W.get("wan14b-480p")
    B, N, H, d = w.B, w.N, w.H, w.d
    C = H * d
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(w.index)
    rnd = lambda *shape: torch.randn(shape, generator=g, device=dev)
    x = (rnd(B * N, C) * 2 + 0.3).to(torch.bfloat16)
    wqc, wqs = sq.w8a8_quantize((rnd(3 * C, C) / C ** 0.5).to(torch.bfloat16))
    woc, wos = sq.w8a8_quantize((rnd(C, C) / C ** 0.5).to(torch.bfloat16))
    bqkv, bo = rnd(3 * C), rnd(C)
    gamma, beta = 1 + 0.2 * rnd(C), 0.1 * rnd(C)
    gq, gk = 1 + 0.1 * rnd(C), 1 + 0.1 * rnd(C)
    y = torch.empty((B * N, 3 * C), dtype=torch.bfloat16, device=dev)
    att = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev)
    z = torch.empty((B * N, C), dtype=torch.bfloat16, device=dev)
    ws1 = torch.empty(sq.w8a8_layernorm_workspace_bytes(B * N, C), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(sq.forward_qknorm_workspace_bytes(B, H, N, d, w.pv, w.q_block), dtype=torch.uint8,
                      device=dev)
    ws3 = torch.empty(sq.w8a8_workspace_bytes(B * N, C), dtype=torch.uint8, device=dev)
    qkv = y.view(B, N, 3, H, d)
    views = [qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)]
    stream = torch.cuda.current_stream(dev)

    def s1():
        sq.w8a8_linear_layernorm(x, wqc, wqs, gamma=gamma, beta=beta, eps=1e-6, bias=bqkv, out=y, workspace=ws1)

    def s2():
        sq.forward_qknorm(*views, gq, gk, 1e-6, scale=w.scale, pv=w.pv, q_block=w.q_block,
                          out=att.permute(0, 2, 1, 3), workspace=ws2)

    def s3():
        sq.w8a8_linear(att.view(B * N, C), woc, wos, bias=bo, out=z, workspace=ws3)

    def step():
        s1()
        s2()
        s3()

    for _ in range(a.warmup):
        step()
    with ClockSampler(_card(torch)) as clocks:
        ms, ms_med, ms_min, _ = _timed(torch, np, dev, stream, step, a.steps)
    t1, t2, t3 = (_timed(torch, np, dev, stream, f, a.steps)[0] for f in (s1, s2, s3))
    ops_qkv, ops_att, ops_out = 2 * B * N * 3 * C * C, w.ops, 2 * B * N * C * C
    ops = ops_qkv + ops_att + ops_out
    tops = ops / (ms * 1e-3) / 1e12
    res = {
        "metric": "DiT attention block TOPS (LayerNorm+W8A8 QKV, q/k-RMSNorm quantized attention, W8A8 out) "
                  "+ % of MI355X INT8 MFMA peak",
        "value": round(tops, 3), "unit": "TOPS", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8+bf16", "data": "synthetic", "pct_int8_peak": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "config": {"workload": "dit-block-wan14b-480p", "B": B, "N": N, "H": H, "d": d, "pv": w.pv,
                   "ops": {"qkv": ops_qkv, "attention": ops_att, "out": ops_out},
                   "stages_ms": {"block_median": round(ms_med, 4), "block_min": round(ms_min, 4),
                                 "layernorm_qkv_projection": round(t1, 4), "qknorm_attention": round(t2, 4),
                                 "out_projection": round(t3, 4)}},
        "roofline": None, "cpu_baseline": None,
        "system": dict(system_info(torch), clocks=clocks.summary()),
    }
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan14b-480p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=None)
    ap.add_argument("--q-block", type=int, default=None,
                    help="Q scale block (1 = one scale per query row); default: the workload's")
    ap.add_argument("--rmsnorm", action="store_true",
                    help="W8A8 workloads: the step is RMSNorm + quantization + GEMM (fused normalization)")
    ap.add_argument("--layernorm", action="store_true",
                    help="W8A8 workloads: the step is LayerNorm + quantization + GEMM (fused normalization)")
    ap.add_argument("--dit-block", action="store_true",
                    help="time the Wan-14B-480p DiT attention block built from the fused pieces "
                         "(LayerNorm+W8A8 QKV, q/k-RMSNorm attention, W8A8 out)")
    ap.add_argument("--qk-norm", action="store_true",
                    help="attention workloads: Q, K, V as views of a fused [B, N, 3, H, d] projection output and "
                         "the step is attention with the per-token q/k RMSNorm fused into the quantization")
    ap.add_argument("--smooth-q", action="store_true",
                    help="attention workloads: Q smoothing per Q block (opts.smooth_q) in the timed forward")
    ap.add_argument("--block-density", type=float, default=None,
                    help="block-sparse attention: fraction of the non-local blocks kept")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (every head is "
              "independent: heads would be split over GPUs with no communication)", file=sys.stderr)
        return 2
    if a.workload.startswith("w8a8-"):
        return bench_w8a8(a)
    if a.dit_block:
        return bench_dit_block(a)

    import numpy as np
    import torch

    import bit_quantized_attention_block_amd as sq
    import workloads as W

    w = W.get(a.workload)
    if a.q_block is not None:
        import dataclasses
        w = dataclasses.replace(w, q_block=a.q_block)
    t0 = time.perf_counter()
    q, k, v, rows = W.gen_inputs(w)
    mask_h = M = None
    ops = w.ops
    if a.block_density is not None:
        mask_h = W.gen_block_mask(w.B, w.H, w.N, a.block_density, seed=w.index)
        ops, processed = sparse_ops(w, mask_h)
    print(f"[bench] generated {w.name} inputs in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    Q, K, V = to(q), to(k), to(v)
    if mask_h is not None:
        M = torch.from_numpy(mask_h).to(dev)
    out = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(sq.workspace_bytes(w.B, w.H, w.N, w.d, w.pv, w.q_block, a.smooth_q), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        sq.forward(Q, K, V, scale=w.scale, pv=w.pv, q_block=w.q_block, out=out, workspace=ws, block_mask=M,
                   smooth_q=a.smooth_q)

    plain_ms = None
    if a.qk_norm:
        # Q, K, V inside one fused projection output [B, N, 3, H, d]; weights of
        # the q and k normalization ~ 1 + N(0, 0.1^2)
        qkv = torch.stack([t.permute(0, 2, 1, 3) for t in (Q, K, V)], dim=2).contiguous()
        qv, kv, vv = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
        g = torch.Generator(device=dev)
        g.manual_seed(w.index)
        Gq, Gk = (1.0 + 0.1 * torch.randn(w.H * w.d, generator=g, device=dev) for _ in range(2))
        wsn = torch.empty(sq.forward_qknorm_workspace_bytes(w.B, w.H, w.N, w.d, w.pv, w.q_block),
                          dtype=torch.uint8, device=dev)

        def plain():
            sq.forward(qv, kv, vv, scale=w.scale, pv=w.pv, q_block=w.q_block, out=out, workspace=ws, block_mask=M)

        for _ in range(2):
            plain()
        plain_ms = _timed(torch, np, dev, stream, plain, a.steps)[0]

        def step():
            sq.forward_qknorm(qv, kv, vv, Gq, Gk, 1e-6, scale=w.scale, pv=w.pv, q_block=w.q_block, out=out,
                              workspace=wsn, block_mask=M)

    def timed(fn, n):
        return _timed(torch, np, dev, stream, fn, n)

    for _ in range(a.warmup):
        step()
    with ClockSampler(_card(torch)) as clocks:
        ms, ms_med, ms_min, t_wall = timed(step, a.steps)
    print(f"[bench] forward {ms:.3f} ms/step (median {ms_med:.3f}, min {ms_min:.3f}; wall "
          f"{t_wall / a.steps * 1e3:.3f}); torch {torch.__version__}, HIP {torch.version.hip}",
          file=sys.stderr, flush=True)

    # ---- the attention kernel alone (one launch per call) on prepared operands
    qi, qs, ki, ks, mu = sq.quantize_qk(Q, K, w.q_block, 64)
    if w.pv == "fp8":
        vc, vs = sq.quantize_v_fp8(V)
        vp = sq.pack_v(vc, "fp8")
    else:
        vs = None
        vp = sq.pack_v(V, "bf16")

    def kern():
        sq.attend_packed(qi, qs, ki, ks, vp, vs, scale=w.scale, pv=w.pv, q_block=w.q_block, out=out,
                            block_mask=M)

    reps = a.kernel_reps or a.steps
    for _ in range(2):
        kern()
    k_ms, k_med, k_min, _ = timed(kern, reps)

    # the quantization/packing stages alone, for the breakdown
    def prep():
        sq.quantize_qk(Q, K, w.q_block, 64)
        if w.pv == "fp8":
            sq.pack_v(sq.quantize_v_fp8(V)[0], "fp8")
        else:
            sq.pack_v(V, "bf16")

    p_ms = timed(prep, reps)[0]

    # fallback ratio: work items that took the exact-max second pass in one
    # forward (the FP8 path rebases every tile and has no such pass)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    sq.forward(Q, K, V, scale=w.scale, pv=w.pv, q_block=w.q_block, out=out, workspace=ws, block_mask=M,
               second_pass_count=cnt, smooth_q=a.smooth_q)
    torch.cuda.synchronize(dev)
    items = w.B * w.H * -(-w.N // 256)
    fallback = {"second_pass_work_items": int(cnt.item()), "work_items": items,
                "ratio": round(int(cnt.item()) / items, 6),
                "what": "work items (one head's 256 query rows) whose row sum reached 2^64 in the one-pass "
                        "softmax and were recomputed with the exact row max" if w.pv == "bf16" else
                        "none by construction: the FP8 path keeps P, O and the row sum relative to the exact "
                        "running max of every tile"}

    tops = ops / (ms * 1e-3) / 1e12
    k_tops = ops / (k_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+bf16" if w.pv == "bf16" else "i8+fp8",
        "data": "synthetic",
        "pct_int8_peak": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "q_block": w.q_block,
                   "k_block": w.k_block, "pv": w.pv, "dist": w.dist,
                   "stages_ms": {"forward_median": round(ms_med, 4), "forward_min": round(ms_min, 4),
                                 "attention_kernel": round(k_ms, 4), "attention_kernel_median": round(k_med, 4),
                                 "attention_kernel_min": round(k_min, 4), "quantize_and_pack": round(p_ms, 4)}},
        "roofline": _at_profiled_clock(
            {"kernel": ATTN_KERNEL[w.pv], "bound": "mfma", "achieved": round(k_tops, 2),
             "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(k_tops / INT8_PEAK_TOPS, 4),
             "peak_mixed": round(mixed_peak(w.pv), 2),
             "frac_mixed": round(k_tops / mixed_peak(w.pv), 4),
             "traffic": _traffic(w.name, ATTN_SRC[w.pv]) if M is None else None,
             "avg_launch_ms": round(k_ms, 4), "ops_per_launch": ops},
            w.name if M is None else "", ATTN_SRC[w.pv]),
    }
    if a.smooth_q:
        res["config"]["smooth_q"] = {
            "step": "Q smoothing per Q block: exact block mean removed before INT8 quantization, returned as a "
                    "logit bias (mean . K', binary32 per block and key) added to the scores"}
    if a.qk_norm:
        res["config"]["qk_norm"] = {
            "layout": "q, k, v as views of a fused [B, N, 3, H, d] projection output",
            "step": "attention with the per-token q/k RMSNorm (over H*d) fused into the quantization",
            "forward_without_norm_ms": round(plain_ms, 4)}
    if M is not None:
        res["metric"] = METRIC.replace("4·B·H·N²·d/s", "4·d·kept query-key pairs/s") + ", block-sparse"
        res["config"]["block_sparse"] = {
            "mask": "128-row x 64-key blocks: local band (keys within 256 rows of the query block) plus a "
                    f"fraction {a.block_density} of the other blocks, seed {w.index}",
            "kept_fraction": round(ops / w.ops, 4),
            "processed_fraction": round(processed / w.ops, 4),
            "dense_equivalent_tops": round(w.ops / (ms * 1e-3) / 1e12, 3)}
        res["roofline"]["processed_ops_per_launch"] = processed
    res["fallback"] = fallback
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        outs = {}
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, rows, mask=mask_h, ops=ops, outs=outs)
        if a.qk_norm or a.smooth_q:
            res["numerics"] = None  # the oracle sample is of the plain forward
        else:
            print("[bench] comparing the sampled rows", file=sys.stderr, flush=True)
            step()
            torch.cuda.synchronize(dev)
            res["numerics"] = numerics(w, q, k, v, out, outs, mask=mask_h)
    else:
        res["cpu_baseline"] = None
        res["numerics"] = None
    res["system"] = system_info(torch)
    res["system"]["clocks"] = clocks.summary()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
