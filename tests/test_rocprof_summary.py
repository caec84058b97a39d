"""Host-side logic of the profile summaries (no GPU, no profiler)."""
import csv
import os

from bit_quantized_attention_block_amd import rocprof_harness as rh


def _trace(tmp_path, rows):
    d = tmp_path / "trace" / "host" / "1"
    d.mkdir(parents=True)
    with open(d / "trace_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Start_Timestamp", "End_Timestamp"], r)))


def test_steady_average_drops_the_first_launch(tmp_path):
    # listed out of order: the first launch is the earliest start, not the first row
    _trace(tmp_path, [("void sqattn::attn_bf16_kernel<128, false, false>(sqattn::AttnParams)", 300, 310),
                      ("void sqattn::attn_bf16_kernel<128, false, false>(sqattn::AttnParams)", 100, 150),
                      ("sqattn::other_kernel(int)", 160, 900),
                      ("void sqattn::attn_bf16_kernel<128, false, false>(sqattn::AttnParams)", 200, 214)])
    is_attn = lambda n: rh._short(n).endswith("attn_bf16_kernel")
    mean, n = rh._steady_ns(str(tmp_path), is_attn)
    assert n == 2 and mean == 12.0


def test_warm_up_launches_are_skipped(tmp_path):
    _trace(tmp_path, [("k(p)", 0, 50), ("k(p)", 100, 140), ("k(p)", 200, 210), ("k(p)", 300, 314)])
    (tmp_path / "trace.log").write_text("[target] warm-up launches: 2\n[target] w: 2 launches done\n")
    n = rh._warm_launches(str(tmp_path), "trace")
    assert n == 2
    assert rh._steady_ns(str(tmp_path), lambda n: True, n) == (12.0, 2)
    assert rh._warm_launches(str(tmp_path), "fetch") == 1  # no log: the first launch only


def test_counter_means_skip_the_warm_up_in_dispatch_order():
    d = {"10": ("k", 5.0), "2": ("k", 100.0), "3": ("copy", 7.0), "11": ("k", 7.0)}
    assert rh._mean_for(d, lambda n: n == "k", 1) == (6.0, 2)
    assert rh._mean_for(d, lambda n: n == "k", 5) == (112.0 / 3, 3)  # fewer left: all of them
    assert rh._mean_for(d, lambda n: n == "copy") == (7.0, 1)


def test_steady_average_needs_two_launches(tmp_path):
    _trace(tmp_path, [("sqattn::w8a8_gemm_kernel(p)", 0, 5)])
    assert rh._steady_ns(str(tmp_path), lambda n: "w8a8_gemm_kernel" in n) is None
    assert rh._steady_ns(str(tmp_path / "nowhere"), lambda n: True) is None


def _csv(path, fields, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))


def test_summarize_end_to_end_on_synthetic_csv(tmp_path):
    """The summary of a W8A8 workload from made-up rocprofv3 output: two
    warm-up launches, two steady ones, the calibration copies; checks the
    figures derived from the counters."""
    import json
    name = "w8a8-qkv-wan14b-480p"
    sp = rh.spec(name)
    out, prof = tmp_path / "out", tmp_path / "prof"
    kern, copy = "sqattn::(anonymous namespace)::w8a8_gemm_kernel(p)", "__amd_rocclr_copyBuffer"
    (out).mkdir()
    (out / "commands.json").write_text(json.dumps(
        {"workload": name, "reps": 2, "outdir": str(out),
         "commands": {p: f"rocprofv3 -d {out}/{p} -- python3 x" for p in ["trace", *rh.COUNTER_PASSES]}}))
    for p in ["trace", *rh.COUNTER_PASSES]:
        (out / (p + ".log")).write_text("[target] warm-up launches: 2\n")
    _csv(out / "trace" / "h" / "trace_kernel_stats.csv",
         ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"],
         [(kern, 4, 12e6, 3e6, 2.8e6, 3.4e6, 90.0), (copy, 3, 1.2e6, 0.4e6, 0.4e6, 0.4e6, 10.0)])
    _csv(out / "trace" / "h" / "trace_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
         [(kern, 0, 3_400_000), (kern, 4_000_000, 7_100_000), (kern, 8_000_000, 10_800_000),
          (kern, 11_000_000, 13_800_000)])
    steady_ns = 2_800_000
    ctr = ["Counter_Name", "Dispatch_Id", "Kernel_Name", "Counter_Value"]
    def pass_rows(vals):
        rows = []
        for c, v in vals.items():
            rows += [(c, i, kern, v) for i in range(1, 5)]
        return rows
    copy_rows = lambda c, v: [(c, 10 + i, copy, v) for i in range(3)]
    _csv(out / "fetch" / "h" / "fetch_counter_collection.csv", ctr,
         pass_rows({"FETCH_SIZE": 1.0e6}) + copy_rows("FETCH_SIZE", (1 << 30) / 2 / 1024))
    _csv(out / "write" / "h" / "write_counter_collection.csv", ctr,
         pass_rows({"WRITE_SIZE": 0.5e6}) + copy_rows("WRITE_SIZE", (1 << 30) / 1024))
    _csv(out / "sq" / "h" / "sq_counter_collection.csv", ctr,
         pass_rows({c: 1000.0 for c in rh.COUNTER_PASSES["sq"]}))
    cycles = 2.0e9 * steady_ns * 1e-9  # 2 GHz per XCD
    _csv(out / "grbm" / "h" / "grbm_counter_collection.csv", ctr,
         pass_rows({"GRBM_GUI_ACTIVE": cycles * 8, "GRBM_COUNT": cycles * 8}))
    mops_i8 = sp["type_ops"]["I8"] / 512
    _csv(out / "mops" / "h" / "mops_counter_collection.csv", ctr,
         pass_rows({"SQ_INSTS_VALU_MFMA_MOPS_I8": mops_i8, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 0.0,
                    "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0, "SQ_INSTS_VALU_MFMA_I8": 100.0,
                    "SQ_INSTS_VALU_MFMA_BF16": 0.0, "SQ_INSTS_VALU_MFMA_F8": 0.0}))
    assert rh.summarize(name, str(out), str(prof)) == 0
    t = json.loads((prof / "kernel_traffic.json").read_text())[name]
    assert t["steady_avg_duration_ns"] == steady_ns
    assert abs(t["sustained_clock_ghz"] - 2.0) < 1e-9
    assert abs(t["read_bytes"] - 2.0 * 1.0e6 * 1024) < 1 and abs(t["write_bytes"] - 0.5e6 * 1024) < 1
    # the operation's I8 ops in 2.8 ms at 2 GHz against 256 CUs x 8138 ops per clock
    want = sp["type_ops"]["I8"] / (5.0e15 / 2.4e9 / 256) / 256 / cycles
    assert abs(t["mfma_utilisation"] - want) < 1e-9
    md = (prof / f"w8a8_gemm_kernel_{name}_profile.md").read_text()
    assert "| I8 | 100 |" in md and "1.0000 |" in md and "Steady: without the 2 warm-up" in md
