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
