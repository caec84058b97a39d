"""Build libsqattn.so (HIP kernels for gfx950 + the C-ABI) in place, and its
checking variant libsqattn_debug.so (-DSQATTN_DEBUG: every wait before a
work-group barrier drains all loads in flight, and the kernels check their
tile and row indices, counting violations in a device word read by
sqattn_debug_violations()).  Tests compare the two bit for bit: a missing
wait in the fast build shows up as a difference.

    python -m bit_quantized_attention_block_amd.build [--jobs N] [--verbose] [--no-debug]

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
LIB_DEBUG = os.path.join(PKG, "libsqattn_debug.so")
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


def _build_one(debug: bool, jobs: int | None, verbose: bool) -> str:
    bdir = BUILD + ("_debug" if debug else "")
    lib = LIB_DEBUG if debug else LIB
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    flags = ["-DSQATTN_DEBUG"] if debug else []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([cc, *COMMON, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(jobs or min(len(cmds), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


def build(jobs: int | None = None, verbose: bool = False, debug: bool = True) -> str:
    """Builds libsqattn.so and (debug) libsqattn_debug.so; returns the former."""
    out = _build_one(False, jobs, verbose)
    if debug:
        _build_one(True, jobs, verbose)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--no-debug", action="store_true", help="skip libsqattn_debug.so")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, not a.no_debug))


if __name__ == "__main__":
    main(sys.argv[1:])
