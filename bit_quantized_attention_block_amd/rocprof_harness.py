"""rocprofv3 harness for the sqattn kernels on one MI355X: the attention
kernels (attention workloads) and the W8A8 GEMM (workloads named w8a8-*).

Sub-commands:

    python -m bit_quantized_attention_block_amd.rocprof_harness target   --workload W [--reps R]
    python -m bit_quantized_attention_block_amd.rocprof_harness collect  --workload W --out DIR
    python -m bit_quantized_attention_block_amd.rocprof_harness summarize --workload W --out DIR
    python -m bit_quantized_attention_block_amd.rocprof_harness bench-trace --workload W --out DIR

`bench-trace` runs rocprofv3 --kernel-trace --stats around bench.py itself and
writes profiles/<kernel>_<workload>_bench_trace.md: the per-kernel durations of
that run next to the HIP-event figures of its bench line.

`target` is the profiled program: seeded inputs of the workload in HBM,
quantize Q/K and pack V once, then R attention kernels back to back -- or, for
a W8A8 workload, quantize x once and R block-scaled GEMMs back to back on
pre-quantized weights -- and, for calibration, three device copies of a 1 GiB
buffer (a plain read + write of known size).

`collect` runs `target` under rocprofv3 in separate passes: kernel trace with
statistics, FETCH_SIZE, WRITE_SIZE, the shader counters of MFMA utilisation,
the GRBM cycle counters, and the matrix ops per operand type
(SQ_INSTS_VALU_MFMA_MOPS_I8 / _BF16 / _F8).  Every pass is its own process under a hard time limit (a pass
that asks for more counters than the hardware has hangs, so each pass holds
only counters that fit one run).

`summarize` turns the CSV output into
  profiles/<kernel>_<workload>_profile.md  kernel durations (rocprofv3 --stats,
                                           and without the first launch), HBM
                                           bytes, MFMA busy and the sustained
                                           shader clock per launch
  profiles/kernel_traffic.json             per-launch HBM bytes of the profiled
                                           kernel, keyed by workload, with a
                                           sha256 over the kernel source and
                                           the headers it includes, as measured.

HBM bytes come from the TCC counters FETCH_SIZE / WRITE_SIZE (KiB per
dispatch), each scaled by the factor that maps the same counter to the known
byte count of the calibration copy.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shlex
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_attention_block_amd", "csrc")
ATTN_SRC = {"bf16": os.path.join(CSRC, "attn_bf16.hip"), "fp8": os.path.join(CSRC, "attn_fp8.hip")}
ATTN_KERNEL = {"bf16": "attn_bf16_kernel", "fp8": "attn_fp8_kernel"}
W8A8_SRC = os.path.join(CSRC, "w8a8.hip")
W8A8_KERNEL = "w8a8_gemm_kernel"


def spec(workload: str) -> dict:
    """The profiled kernel of a workload: name, source, operation count, title."""
    sys.path.insert(0, ROOT)
    if workload.startswith("w8a8-"):
        from workloads import linear as WL
        w = WL.get_linear(workload)
        return {"w": w, "kind": "w8a8", "kernel": W8A8_KERNEL, "src": W8A8_SRC, "ops": w.ops,
                "ops_text": "2 M N K", "type_ops": {"I8": w.ops},
                "title": f"{w.name} (M={w.M}, N={w.N}, K={w.K}, bf16 output, bias)"}
    import workloads as W
    w = W.get(workload)
    return {"w": w, "kind": "attn", "kernel": ATTN_KERNEL[w.pv], "src": ATTN_SRC[w.pv], "ops": w.ops,
            "ops_text": "4 B H N^2 d", "type_ops": {"I8": w.ops / 2, ("BF16" if w.pv == "bf16" else "F8"): w.ops / 2},
            "title": f"{w.name} (B={w.B}, H={w.H}, N={w.N}, d={w.d}, P.V {w.pv})"}
COPY_BYTES = 1 << 30
WARM_SECONDS = 0.25
N_XCD = 8                   # accelerator complex dies of the MI355X (one GRBM each)
INT8_PEAK_OPS = 5.0e15      # dense INT8 matrix peak quoted for the MI355X ...
PEAK_CLOCK_GHZ = 2.4        # ... at this shader clock
COPY_REPS = 3

COUNTER_PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "sq": ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
           "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT"],
    "grbm": ["GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    "mops": ["SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
             "SQ_INSTS_VALU_MFMA_I8", "SQ_INSTS_VALU_MFMA_BF16", "SQ_INSTS_VALU_MFMA_F8"],
}
# dense matrix peaks quoted for the MI355X at 2.4 GHz, ops/s, per operand type
# of the MOPS counters (F8 counts the E4M3 scaled MFMA)
TYPE_PEAK_OPS = {"I8": 5.0e15, "BF16": 2.5e15, "F8": 5.0e15}


# ---------------------------------------------------------------------------
# target
# ---------------------------------------------------------------------------
def run_target(workload: str, reps: int) -> None:
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import bit_quantized_attention_block_amd as sq
    import workloads as W

    sp = spec(workload)
    w = sp["w"]
    dev = torch.device("cuda:0")
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    if sp["kind"] == "w8a8":
        from workloads import linear as WL
        X, Wt = to(WL.gen_x(w)), to(WL.gen_w(w))
        bias = torch.from_numpy(WL.gen_bias(w)).to(dev)
        wc, ws = sq.w8a8_quantize(Wt)
        del Wt
        y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        xc, xs = sq.w8a8_quantize(X)
        launch = lambda: sq.w8a8_gemm(xc, xs, wc, ws, bias=bias, out=y)
    else:
        q, k, v, _ = W.gen_inputs(w)
        Q, K, V = to(q), to(k), to(v)
        out = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        qi, qs, ki, ks, _mu = sq.quantize_qk(Q, K, w.q_block, w.k_block)
        if w.pv == "fp8":
            vc, vs = sq.quantize_v_fp8(V)
            vp = sq.pack_v(vc, "fp8")
        else:
            vs, vp = None, sq.pack_v(V, "bf16")
        launch = lambda: sq.attend_packed(qi, qs, ki, ks, vp, vs, scale=w.scale, pv=w.pv, q_block=w.q_block,
                                          out=out)
    torch.cuda.synchronize()
    # Warm-up: the profiled kernel itself for about WARM_SECONDS, so that the
    # shader clock has left its idle level (the summary leaves these launches
    # out of the steady figures), then the profiled launches back to back, as
    # the bench times them.
    n_warm, t0 = 0, time.time()
    while time.time() - t0 < WARM_SECONDS:
        launch()
        n_warm += 1
        if n_warm % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"[target] warm-up launches: {n_warm}", flush=True)
    for _ in range(reps):
        launch()
    torch.cuda.synchronize()
    print(f"[target] {w.name}: {reps} launches done", flush=True)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[target] calibration copies of {COPY_BYTES} bytes done", flush=True)


# ---------------------------------------------------------------------------
# collect
# ---------------------------------------------------------------------------
def _target_cmd(workload: str, reps: int) -> list[str]:
    return [sys.executable, "-m", "bit_quantized_attention_block_amd.rocprof_harness", "target",
            "--workload", workload, "--reps", str(reps)]


def _rocprof(args: list[str], outdir: str, name: str, workload: str, reps: int, limit: int) -> list[str]:
    cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", *args, "-d", os.path.join(outdir, name), "-o", name,
           "--output-format", "csv", "--", *_target_cmd(workload, reps)]
    return cmd


def collect(workload: str, outdir: str, reps: int) -> int:
    outdir = os.path.abspath(outdir)
    os.makedirs(outdir, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    passes = [("trace", ["--kernel-trace", "--stats"], 300)]
    passes += [(n, ["--pmc", *c], 240) for n, c in COUNTER_PASSES.items()]
    commands = {}
    for name, args, limit in passes:
        cmd = _rocprof(args, outdir, name, workload, reps, limit)
        commands[name] = " ".join(shlex.quote(c) for c in cmd)
        print(f"[collect] pass {name}: {commands[name]}", flush=True)
        t0 = time.time()
        with open(os.path.join(outdir, name + ".log"), "w") as log:
            rc = subprocess.call(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT)
        print(f"[collect] pass {name} rc={rc} in {time.time() - t0:.1f} s", flush=True)
        if rc != 0:
            return rc
    with open(os.path.join(outdir, "commands.json"), "w") as f:
        json.dump({"workload": workload, "reps": reps, "outdir": outdir, "commands": commands}, f, indent=1)
    return 0


# ---------------------------------------------------------------------------
# summarize
# ---------------------------------------------------------------------------
def _rows(outdir: str, name: str, suffix: str):
    files = glob.glob(os.path.join(outdir, name, "**", f"*{suffix}"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, value)} for one counter (values summed over
    the counter's instances)."""
    d = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        name, val = d.get(key, (r["Kernel_Name"], 0.0))
        d[key] = (name, val + float(r["Counter_Value"]))
    return d


def _mean_for(d, match, skip: int = 0):
    """Mean over the matching dispatches in dispatch order, without the first
    `skip` of them (all of them if fewer are left)."""
    keys = sorted(d, key=lambda k: int(k) if str(k).isdigit() else str(k))
    vals = [d[k][1] for k in keys if match(d[k][0])]
    if len(vals) > skip:
        vals = vals[skip:]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def _short(name: str) -> str:
    """Kernel name without namespaces' "(anonymous namespace)" part, argument
    list or template arguments."""
    return name.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0]


def _shown(name: str) -> str:
    """Kernel name as listed: without the "(anonymous namespace)" part and the
    argument list, with template arguments (they tell instantiations apart)."""
    n = name.replace("(anonymous namespace)::", "")
    return n[:n.index(">") + 1] if "<" in n.split("(")[0] else n.split("(")[0]


def _includes(path):
    """The sources a kernel file compiles: the file and, recursively, the
    headers it includes by a quoted name from its own directory, sorted."""
    seen, todo = set(), [os.path.abspath(path)]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(f):
            continue
        seen.add(f)
        with open(f) as fh:
            for line in fh:
                t = line.strip()
                if t.startswith("#include \""):
                    todo.append(os.path.join(os.path.dirname(f), t.split('"')[1]))
    return sorted(seen)


def source_key(path):
    """sha256 over the kernel file and every header it includes (name and
    bytes of each, in sorted order): a counter summary is only valid for the
    code it was taken on."""
    h = hashlib.sha256()
    for f in _includes(path):
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _warm_launches(outdir: str, name: str) -> int:
    """Warm-up launches the target reported in a pass's log (1 if absent: the
    first launch of the process is left out in any case)."""
    try:
        with open(os.path.join(outdir, name + ".log")) as f:
            for line in f:
                if line.startswith("[target] warm-up launches:"):
                    return max(1, int(line.split(":")[1]))
    except (OSError, ValueError):
        pass
    return 1


def _steady_ns(outdir: str, match, skip: int = 1):
    """(mean duration in ns, count) of the matching dispatches of the kernel
    trace without the first `skip`, or None when none are left."""
    rows = [r for r in _rows(outdir, "trace", "kernel_trace.csv") if match(r.get("Kernel_Name", ""))]
    try:
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows[skip:]]
    except (KeyError, ValueError):
        return None
    return (sum(d) / len(d), len(d)) if d else None


def summarize(workload: str, outdir: str, profiles: str) -> int:
    sp = spec(workload)
    w = sp["w"]
    kname = sp["kernel"]
    is_attn = lambda n: _short(n).endswith(kname)
    is_copy = lambda n: "copybuffer" in n.lower()  # the device-to-device copy of torch copy_
    with open(os.path.join(outdir, "commands.json")) as f:
        meta = json.load(f)

    # kernel durations
    stats = _rows(outdir, "trace", "kernel_stats.csv")
    stat_lines = ["| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    attn_avg_ns = None
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        short = _short(name)
        stat_lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                          f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                          f"{float(r['Percentage']):.1f}% |")
        if is_attn(name):
            attn_avg_ns = float(r["AverageNs"])

    # counters
    fetch = _per_dispatch(_rows(outdir, "fetch", "counter_collection.csv"), "FETCH_SIZE")
    write = _per_dispatch(_rows(outdir, "write", "counter_collection.csv"), "WRITE_SIZE")
    sqr = _rows(outdir, "sq", "counter_collection.csv")
    grbm = _rows(outdir, "grbm", "counter_collection.csv")
    # the kernel's counters over its launches after the target's warm-up
    f_attn, n_attn = _mean_for(fetch, is_attn, _warm_launches(outdir, "fetch"))
    w_attn, _ = _mean_for(write, is_attn, _warm_launches(outdir, "write"))
    f_copy, n_copy = _mean_for(fetch, is_copy)
    w_copy, _ = _mean_for(write, is_copy)
    if None in (f_attn, w_attn, f_copy, w_copy) or not f_copy or not w_copy:
        print("[summarize] missing counter data", file=sys.stderr)
        return 1
    f_scale = COPY_BYTES / (f_copy * 1024.0)   # bytes per counted byte
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    read_b = f_attn * 1024.0 * f_scale
    write_b = w_attn * 1024.0 * w_scale
    traffic = read_b + write_b

    sq_vals = {}
    for c in COUNTER_PASSES["sq"]:
        v, _ = _mean_for(_per_dispatch(sqr, c), is_attn, _warm_launches(outdir, "sq"))
        sq_vals[c] = v
    for c in COUNTER_PASSES["grbm"]:
        v, _ = _mean_for(_per_dispatch(grbm, c), is_attn, _warm_launches(outdir, "grbm"))
        sq_vals[c] = v
    mops_rows = _rows(outdir, "mops", "counter_collection.csv")
    mops = {}
    for c in COUNTER_PASSES["mops"]:
        v, _ = _mean_for(_per_dispatch(mops_rows, c), is_attn, _warm_launches(outdir, "mops"))
        mops[c] = v

    ops = sp["ops"]
    lines = [f"# `{kname}` on {sp['title']}", "",
             f"Made by `python -m bit_quantized_attention_block_amd.rocprof_harness collect --workload {w.name} "
             f"--out <out>` on one MI355X, which runs these passes from /tmp with TMPDIR=/tmp and the "
             f"repository root on PYTHONPATH:", ""]
    rec_out = meta.get("outdir") or shlex.split(meta["commands"]["trace"]).__getitem__(
        shlex.split(meta["commands"]["trace"]).index("-d") + 1).rsplit("/", 1)[0]
    for name, cmd in meta["commands"].items():
        cmd = cmd.replace(rec_out, "<out>").replace(sys.executable, "python3")
        cmd = " ".join("python3" if c.endswith("/python") or c.endswith("/python3") else c for c in cmd.split(" "))
        lines += [f"- {name}: `{cmd}`"]
    lines += ["", f"Summarized with `python -m bit_quantized_attention_block_amd.rocprof_harness summarize "
                  f"--workload {w.name} --out <dir>`.", "",
              "## Kernel durations (rocprofv3 --kernel-trace --stats)", ""] + stat_lines
    if attn_avg_ns:
        lines += ["", f"`{kname}` average: {attn_avg_ns / 1e6:.3f} ms -> "
                      f"{ops / (attn_avg_ns * 1e-9) / 1e12:.1f} TOPS ({sp['ops_text']} / t)."]
    n_warm = _warm_launches(outdir, "trace")
    steady = _steady_ns(outdir, is_attn, n_warm)
    if steady:
        lines += [f"Steady: without the {n_warm} warm-up launch(es) of the process (code loading, cold caches, "
                  f"the shader clock leaving its idle level), over the other {steady[1]} launches of the kernel "
                  f"trace: {steady[0] / 1e6:.3f} ms -> {ops / (steady[0] * 1e-9) / 1e12:.1f} TOPS.  The counters "
                  f"below are averaged over the launches after each pass's own warm-up."]
    lines += ["", f"## HBM traffic per `{kname}` launch (TCC FETCH_SIZE / WRITE_SIZE)", "",
              f"- calibration: device copy of {COPY_BYTES} bytes, {n_copy} dispatches; FETCH_SIZE reads "
              f"{f_copy:.0f} KiB, WRITE_SIZE {w_copy:.0f} KiB per copy -> scale {f_scale:.4f} (read), "
              f"{w_scale:.4f} (write)",
              f"- `{kname}` ({n_attn} dispatches): FETCH_SIZE {f_attn:.0f} KiB, WRITE_SIZE {w_attn:.0f} KiB",
              f"- scaled: read {read_b / 1e9:.3f} GB, write {write_b / 1e9:.3f} GB, total {traffic / 1e9:.3f} GB "
              f"per launch"]
    if attn_avg_ns:
        lines += [f"- at the traced average duration: {traffic / (attn_avg_ns * 1e-9) / 1e9:.0f} GB/s "
                  f"(HBM peak 8000 GB/s)"]
    lines += ["", f"## Shader counters per `{kname}` launch (sums over the device)", ""]
    for c, v in sq_vals.items():
        lines += [f"- {c}: {v:.4g}" if v is not None else f"- {c}: n/a"]
    dur_ns = steady[0] if steady else attn_avg_ns
    clock_ghz = None
    if sq_vals.get("GRBM_GUI_ACTIVE") and dur_ns:
        # GRBM counts shader-clock cycles in each of the 8 XCDs (summed over them)
        clock_ghz = sq_vals["GRBM_GUI_ACTIVE"] / N_XCD / (dur_ns * 1e-9) / 1e9
        frac = ops / (dur_ns * 1e-9) / (INT8_PEAK_OPS * clock_ghz / PEAK_CLOCK_GHZ)
        lines += ["", f"Sustained shader clock: GRBM_GUI_ACTIVE / {N_XCD} XCDs / kernel time "
                      f"({'steady' if steady else 'traced'} average) = {clock_ghz:.3f} GHz; at that clock the "
                      f"INT8 matrix peak is {INT8_PEAK_OPS * clock_ghz / PEAK_CLOCK_GHZ / 1e12:.0f} TOPS and the "
                      f"kernel reaches {frac:.3f} of it ({frac * clock_ghz / PEAK_CLOCK_GHZ:.3f} of the "
                      f"{INT8_PEAK_OPS / 1e12:.0f} TOPS quoted at {PEAK_CLOCK_GHZ} GHz)."]
    mfma_util = None
    if any(v is not None for v in mops.values()):
        lines += ["", f"## Matrix-core work per `{kname}` launch (SQ_INSTS_VALU_MFMA_MOPS_*: ops / 512)", "",
                  "| operand type | instructions | ops counted | ops of the operation | counted / operation |",
                  "|---|---|---|---|---|"]
        need_cycles = 0.0  # CU-cycles the counted ops need at the quoted per-clock peaks
        for t in ("I8", "BF16", "F8"):
            m, n = mops.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}"), mops.get(f"SQ_INSTS_VALU_MFMA_{t}")
            if m is None:
                continue
            got, want = m * 512.0, sp["type_ops"].get(t, 0.0)
            lines += [f"| {t} | {n:.4g} | {got:.4g} | {want:.4g} | " + (f"{got / want:.4f} |" if want else "— |")]
            need_cycles += got / (TYPE_PEAK_OPS[t] / PEAK_CLOCK_GHZ / 1e9 / 256)
        if sq_vals.get("GRBM_GUI_ACTIVE"):
            cycles = sq_vals["GRBM_GUI_ACTIVE"] / N_XCD  # per XCD, i.e. per CU
            mfma_util = need_cycles / 256 / cycles
            lines += ["", f"At the quoted per-clock peaks (I8 and F8 {TYPE_PEAK_OPS['I8'] / 2.4e9 / 256:.0f}, "
                          f"BF16 {TYPE_PEAK_OPS['BF16'] / 2.4e9 / 256:.0f} ops per clock per CU) the counted ops "
                          f"keep the matrix cores of the 256 CUs busy {need_cycles / 256:.4g} cycles of the "
                          f"kernel's {cycles:.4g}: matrix-core utilisation {mfma_util:.3f}."]
    if sq_vals.get("SQ_VALU_MFMA_BUSY_CYCLES") and sq_vals.get("SQ_BUSY_CYCLES"):
        lines += ["", "SQ_VALU_MFMA_BUSY_CYCLES is counted per SIMD; SQ_BUSY_CYCLES per shader engine "
                      "(32 engines, 32 SIMDs each): MFMA busy fraction = "
                      f"{sq_vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (sq_vals['SQ_BUSY_CYCLES'] * 32):.3f}."]
    os.makedirs(profiles, exist_ok=True)
    stem = f"{kname}_{w.name}"
    with open(os.path.join(profiles, stem + "_profile.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    tf = os.path.join(profiles, "kernel_traffic.json")
    try:
        with open(tf) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {}
    allt[w.name] = {"kernel": kname, "src_key": source_key(sp["src"]),
                    "src_files": [os.path.basename(f) for f in _includes(sp["src"])],
                    "bytes_per_launch": round(traffic),
                    "read_bytes": round(read_b), "write_bytes": round(write_b),
                    "fetch_kib": f_attn, "write_kib": w_attn, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
                    "copy_bytes": COPY_BYTES, "avg_duration_ns": attn_avg_ns,
                    "steady_avg_duration_ns": steady[0] if steady else None,
                    "sustained_clock_ghz": clock_ghz, "mfma_utilisation": mfma_util}
    with open(tf, "w") as f:
        json.dump(allt, f, indent=1, sort_keys=True)
    print("\n".join(lines))
    return 0


# ---------------------------------------------------------------------------
# bench-trace: the kernel trace of bench.py itself
# ---------------------------------------------------------------------------
def bench_trace(workload: str, outdir: str, profiles: str, steps: int, warmup: int, extra: str = "",
                tag: str = "") -> int:
    """rocprofv3 --kernel-trace --stats around `python3 bench.py` (the same
    command that produces the bench line, without the CPU baseline), then
    profiles/<kernel>_<workload>_bench_trace.md with the per-kernel durations
    next to the bench line's own HIP-event figures from that run."""
    sp = spec(workload)
    w = sp["w"]
    kname = sp["kernel"]
    outdir = os.path.abspath(outdir)
    os.makedirs(outdir, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    bench = ["python3", os.path.join(ROOT, "bench.py"), "--workload", w.name, "--steps", str(steps),
             "--warmup", str(warmup), "--no-cpu-baseline", *shlex.split(extra)]
    wname = w.name + (f"-{tag}" if tag else "")
    cmd = ["timeout", "-s", "KILL", "600", "rocprofv3", "--kernel-trace", "--stats", "-d",
           os.path.join(outdir, "bench_trace"), "-o", "bench_trace", "--output-format", "csv", "--", *bench]
    print(f"[bench-trace] {' '.join(shlex.quote(c) for c in cmd)}", flush=True)
    with open(os.path.join(outdir, "bench_trace.json"), "w") as out, \
            open(os.path.join(outdir, "bench_trace.log"), "w") as log:
        rc = subprocess.call(cmd, cwd="/tmp", env=env, stdout=out, stderr=log)
    print(f"[bench-trace] rc={rc}", flush=True)
    if rc != 0:
        return rc
    return bench_trace_summary(workload, outdir, profiles, bench, extra, tag)


def bench_trace_summary(workload: str, outdir: str, profiles: str, bench: list, extra: str = "",
                        tag: str = "") -> int:
    """profiles/<kernel>_<workload>[-tag]_bench_trace.md from the output of a
    bench-trace run in outdir (bench: the traced bench.py command)."""
    sp = spec(workload)
    w = sp["w"]
    kname = sp["kernel"]
    wname = w.name + (f"-{tag}" if tag else "")
    with open(os.path.join(outdir, "bench_trace.json")) as f:
        line = [l for l in f.read().splitlines() if l.startswith("{")][-1]
    res = json.loads(line)
    stats = _rows(outdir, "bench_trace", "kernel_stats.csv")
    is_attn = lambda n: _short(n).endswith(kname)
    rows = ["| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    attn = None
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        rows.append(f"| `{_shown(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                    f"{float(r['Percentage']):.1f}% |")
        if is_attn(r["Name"]):
            attn = float(r["AverageNs"]) / 1e6
    shown = " ".join(c if not c.startswith(ROOT) else c.replace(ROOT, ".") for c in bench)
    lines = [f"# `{kname}` on {wname}: kernel trace of the bench command", "",
             f"Command (from /tmp with TMPDIR=/tmp): `rocprofv3 --kernel-trace --stats -d <out>/bench_trace "
             f"-o bench_trace --output-format csv -- {shown}`, run by `python -m "
             f"bit_quantized_attention_block_amd.rocprof_harness bench-trace --workload {w.name}"
             + (f" --extra='{extra}' --tag {tag}" if extra else "") + "`.", "",
             "## Kernel durations (rocprofv3 --kernel-trace --stats)", ""] + rows + [""]
    k_ev = res["roofline"]["avg_launch_ms"]
    lines += [f"- `{kname}`, rocprofv3 average over all its launches in the run: {attn:.4f} ms",
              f"- `{kname}`, the bench line's HIP-event average (same run): {k_ev:.4f} ms "
              f"({100.0 * (attn - k_ev) / k_ev:+.2f}%)",
              f"- one step (the bench line's `ms_per_step`): {res['ms_per_step']:.4f} ms, "
              f"value {res['value']} {res['unit']}", "",
              "Bench line of the traced run:", "", "```", line, "```"]
    os.makedirs(profiles, exist_ok=True)
    with open(os.path.join(profiles, f"{kname}_{wname}_bench_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("cmd", choices=["target", "collect", "summarize", "bench-trace"])
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b-480p")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--out", default=os.path.join(ROOT, "rocprof_out"))
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--extra", default="", help="bench-trace: further bench.py options (one string)")
    ap.add_argument("--tag", default="", help="bench-trace: suffix of the workload in the summary's name")
    a = ap.parse_args(argv)
    if a.cmd == "target":
        run_target(a.workload, a.reps)
        return 0
    if a.cmd == "collect":
        return collect(a.workload, a.out, a.reps)
    if a.cmd == "bench-trace":
        return bench_trace(a.workload, a.out, a.profiles, a.steps, a.warmup, a.extra, a.tag)
    return summarize(a.workload, a.out, a.profiles)


if __name__ == "__main__":
    sys.exit(main())
