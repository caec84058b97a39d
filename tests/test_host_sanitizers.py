"""The C-ABI layer (csrc/api.cpp) on the host under AddressSanitizer and
UndefinedBehaviorSanitizer.

tests/host/api_harness.cpp links api.cpp with recorders in place of the HIP
runtime calls and the kernel launchers (nothing runs on a GPU and no pointer
is dereferenced): each launcher records the byte ranges its kernels read and
write.  The harness checks argument rejection (status, message, nothing
enqueued or allocated), that every accepted call's ranges stay inside the
caller's buffers, the workspace, the static scratch or the library's own
stream-ordered allocations (freed again), that workspace regions of
different launches do not overlap and are written before they are read, and
the *_workspace_bytes sizes (exactly enough; 256 bytes less refused), over
ragged and maximal sizes.  The sanitizers make any host out-of-bounds access,
leak, or signed overflow in the size arithmetic fatal.  The helpers of
exact.h / e4m3.h run under the same flags in test_exact_host.py."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_attention_block_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIP_INCLUDE = "/opt/rocm/include"
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if not shutil.which("g++") or not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path_factory.mktemp("api") / "api_harness")
    subprocess.run(["g++", "-std=c++17", *SANITIZE, "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", CSRC,
                    "-I", INCLUDE, os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "host",
                                                                               "api_harness.cpp"),
                    "-o", exe], check=True)
    return exe


def test_api_layer_under_sanitizers(harness):
    r = subprocess.run([harness], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    n, fails = r.stdout.split()[0], r.stdout.split()[2]
    assert int(n) > 500 and fails == "0", r.stdout
