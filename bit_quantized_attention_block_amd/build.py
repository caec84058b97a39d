"""Build libsqattn.so (HIP kernels for gfx950 + the C-ABI) in place.

    python -m bit_quantized_attention_block_amd.build [--jobs N] [--verbose]

Every source is compiled with hipcc for gfx950 only; packed-FP32 VALU forms
are disabled (-packed-fp32-ops) and no fast-math flag is used, so binary32
division and subtraction stay IEEE (the quantizers depend on it).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsqattn.so")
SOURCES = ["api.cpp", "prep.hip", "attn_bf16.hip", "attn_fp8.hip", "w8a8.hip", "norm.hip", "static_scratch.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([cc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(jobs or min(len(cmds), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main(sys.argv[1:])
