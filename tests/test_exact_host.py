"""CPU tests of the HIP path's exact-arithmetic helpers, built for the host.

``csrc/exact.h`` (the 192-bit K-mean accumulator and its correctly rounded
division) and ``csrc/e4m3.h`` (the E4M3 encoder of the V quantizer) compile
for host and device.  Here they are built with g++ into a small driver and
compared bit for bit with the oracle on adversarial inputs.  The oracle and
these helpers share no code."""
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import fp, quant
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_attention_block_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>
#include "exact.h"
#include "e4m3.h"
using namespace sqattn;
int main(int argc, char** argv) {
  char mode[16];
  if (scanf("%15s", mode) != 1) return 2;
  if (!strcmp(mode, "mean") || !strcmp(mode, "meanf")) {
    const bool f64 = mode[4] == 'f';
    int cols; if (scanf("%d", &cols) != 1) return 2;
    for (int c = 0; c < cols; ++c) {
      int n; if (scanf("%d", &n) != 1) return 2;
      Acc192 acc; acc192_zero(acc); int64_t win = 0; double wf = 0.0; bool bad = false;
      for (int i = 0; i < n; ++i) { unsigned b; if (scanf("%u", &b) != 1) return 2;
        if (f64) {  // the GPU kernel's order: binary64 window, the rest outside it
          wf += kmean_window_value(b);
          if (!kmean_in_window(b)) bad |= kmean_add_outside(acc, b);
          if (i % KMEAN_F64_ADDS == KMEAN_F64_ADDS - 1) kmean_flush_f64(acc, wf);
        } else {
          bad |= kmean_accumulate(acc, win, b);
          if ((i & 1023) == 1023) kmean_flush_window(acc, win);
        } }
      kmean_flush_window(acc, win);
      kmean_flush_f64(acc, wf);
      float m = acc192_mean_f32(acc, (uint32_t)n);
      uint32_t u; memcpy(&u, &m, 4);
      printf("%d %u %llu %llu %llu\n", bad ? 1 : 0, u, (unsigned long long)acc.w0, (unsigned long long)acc.w1,
             (unsigned long long)acc.w2);
    }
  } else {
    int n; if (scanf("%d", &n) != 1) return 2;
    for (int i = 0; i < n; ++i) { unsigned u; if (scanf("%u", &u) != 1) return 2;
      float y; memcpy(&y, &u, 4); printf("%u\n", e4m3_encode_f32(y)); }
  }
  return 0;
}
"""


# the driver is built twice: optimised, and for the host sanitizers
# (AddressSanitizer + UndefinedBehaviorSanitizer, any report fatal), so that
# every case below also runs the helpers under both
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
SAN_ENV = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(scope="module", params=["O2", "sanitize"])
def driver(request, tmp_path_factory):
    d = tmp_path_factory.mktemp("exact")
    src = d / "drv.cpp"
    src.write_text(DRIVER)
    exe = d / "drv"
    flags = ["-O2"] if request.param == "O2" else SANITIZE
    subprocess.run(["g++", *flags, "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return str(exe)


def _run(exe, text):
    r = subprocess.run([exe], input=text, capture_output=True, text=True, env=SAN_ENV)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-2000:]
    return r.stdout.split()


def _columns():
    rng = np.random.default_rng(17)
    cols = []
    # workload-like columns: N(0,1) + offset, tails, many sizes
    for n in (1, 2, 3, 64, 129, 1000, 32760):
        cols.append(W.f32_to_bf16_bits((rng.standard_normal(n) + rng.normal(0, 1.4)).astype(np.float32)))
    # wide exponent spread, subnormal bf16 values, exact cancellation, zeros
    x = rng.standard_normal(5000) * np.exp2(rng.uniform(-140, 30, 5000))
    cols.append(W.f32_to_bf16_bits(x.astype(np.float32)))
    cols.append(W.f32_to_bf16_bits(np.float32([2.0 ** 30, 1.0, -(2.0 ** 30), 2.0 ** -130])))
    cols.append(np.zeros(77, np.uint16))
    cols.append(np.uint16([0x0001, 0x8001, 0x0001]))          # bf16 subnormals only
    half = W.f32_to_bf16_bits(rng.standard_normal(300).astype(np.float32))
    cols.append(np.concatenate([half, half ^ np.uint16(0x8000)]))
    cols.append(W.f32_to_bf16_bits(np.full(999, 3.0e-5, np.float32)))
    return cols


def _window_edge_columns():
    """Columns at the edges of the binary64 window: 64 in-window values of the
    largest magnitude (16320 = 255 * 2^6) beside the smallest (2^-26), so a
    flushed sum needs all 53 bits; values one binade either side of the
    window; long columns of mixed signs."""
    big, small = np.float32(16320.0), np.float32(129 * 2.0 ** -33)   # 129 * 2^-33: the window's unit is 2^-33
    cols = [np.tile(np.float32([big, small]), 64), np.float32(([big] * 63 + [small]) * 9),
            np.tile(np.float32([big, -small, -big, small, big]), 51),
            np.float32([2.0 ** 14, 2.0 ** -27, 16320.0, 2.0 ** -26, -(2.0 ** 14) * 1.5, 1.0] * 40)]
    rng = np.random.default_rng(5)
    x = np.where(rng.random(20000) < 0.5, -1.0, 1.0) * np.exp2(rng.integers(-26, 14, 20000)) * rng.integers(128, 256, 20000) / 128
    cols.append(x.astype(np.float32))
    return [W.f32_to_bf16_bits(c) for c in cols]


@pytest.mark.parametrize("mode", ["mean", "meanf"])
def test_kmean_host_build_matches_oracle(driver, mode):
    """mean: the 64-bit integer window; meanf: the binary64 window the GPU
    kernel adds into (flushed every KMEAN_F64_ADDS values)."""
    cols = _columns() + _window_edge_columns()
    text = "%s %d\n" % (mode, len(cols)) + "".join(
        "%d %s\n" % (c.size, " ".join(str(int(v)) for v in c)) for c in cols)
    out = _run(driver, text)
    for i, c in enumerate(cols):
        bad, bits, w0, w1, w2 = (int(v) for v in out[5 * i: 5 * i + 5])
        assert bad == 0
        ref = quant.kmean_exact(c.reshape(-1, 1))[0]
        assert bits == int(np.float32(ref).view(np.uint32)), (i, bits, ref)
        # the accumulator holds the exact sum in units of 2^-133 (two's complement)
        units = sum(int(np.ldexp(float(v), 133)) for v in W.bf16_bits_to_f32(c).astype(np.float64))
        assert (w0 | (w1 << 64) | (w2 << 128)) == units % (1 << 192), i


@pytest.mark.parametrize("mode", ["mean", "meanf"])
def test_kmean_host_build_flags_out_of_range(driver, mode):
    cols = [W.f32_to_bf16_bits(np.float32([1.0, 2.0 ** 33])), W.f32_to_bf16_bits(np.float32([2.0 ** 32, -1.0])),
            np.uint16([0x7F80, 0x3F80])]
    text = "%s 3\n" % mode + "".join("%d %s\n" % (c.size, " ".join(str(int(v)) for v in c)) for c in cols)
    out = _run(driver, text)
    assert [int(out[0]), int(out[5]), int(out[10])] == [1, 0, 1]


def test_e4m3_host_build_matches_oracle(driver):
    rng = np.random.default_rng(23)
    y = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-16, 9.5, 200_000))).astype(np.float32)
    pos = fp.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    extra = np.float32([0.0, -0.0, 448.0, 463.99, 464.0, 500.0, 1e30, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11,
                        1e-40, -1e-40])
    y = np.concatenate([y, mids, -mids, pos.astype(np.float32), extra])
    text = "e4m3 %d\n%s\n" % (y.size, " ".join(str(int(u)) for u in y.view(np.uint32)))
    got = np.array([int(s) for s in _run(driver, text)], np.uint8)
    assert np.array_equal(got, fp.e4m3_encode(y))


def test_quotient_shortcut_matches_division():
    """The quantizers' rne(fl32(a/s)) shortcut (csrc/prep.hip rne_quotient),
    emulated in IEEE float32 with numpy: q = RN(a * RN(1/s)), the division
    where q lies within 2^-15 of a half-integer.  It must equal rint of the
    correctly rounded quotient on every value of a block against its own
    scale s = fl32(amax/127): random values, exact ties k + 1/2, and the
    values one ulp either side of a tie."""
    import numpy as np
    rng = np.random.default_rng(12)
    f = np.float32
    amax = (np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-100, 100, 4000))).astype(f)
    s = (amax / f(127)).astype(f)
    y = (f(1) / s).astype(f)
    cols = [rng.uniform(-1, 1, (4000, 400)).astype(f) * amax[:, None]]
    k = rng.integers(-127, 127, (4000, 60)).astype(f)
    tie = ((k + f(0.5)) * s[:, None]).astype(f)                      # often exactly representable
    cols += [tie, np.nextafter(tie, f(np.inf)), np.nextafter(tie, f(-np.inf)), amax[:, None], -amax[:, None]]
    a = np.concatenate(cols, axis=1)
    a = np.clip(a, -amax[:, None], amax[:, None])
    exact = np.rint((a / s[:, None]).astype(f))
    q = (a * y[:, None]).astype(f)
    r = np.rint(q)
    near = np.abs((q - r).astype(f)) > f(0.5 - 2.0 ** -15)
    short = np.where(near, exact, r)
    assert np.array_equal(short, exact)
    assert near[:, :400].mean() < 1e-3     # on the random values the division is the exception
