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


def test_steady_average_needs_two_launches(tmp_path):
    _trace(tmp_path, [("sqattn::w8a8_gemm_kernel(p)", 0, 5)])
    assert rh._steady_ns(str(tmp_path), lambda n: "w8a8_gemm_kernel" in n) is None
    assert rh._steady_ns(str(tmp_path / "nowhere"), lambda n: True) is None
