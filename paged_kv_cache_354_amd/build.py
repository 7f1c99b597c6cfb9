"""Builds libpagedkv.so (HIP kernels + C ABI + host block manager) for gfx950.

Usage: ``python -m paged_kv_cache_354_amd.build`` (also called by
``__graft_entry__.build``).  The library is written next to this file.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedkv.so")
SOURCES = [
    "csrc/pa_status.cpp",
    "csrc/block_manager.cpp",
    "csrc/pa_cache_ops.hip",
    "csrc/pa_decode.hip",
    "csrc/pa_decode_gqa.hip",
    "csrc/pa_prefill.hip",
]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpagedkv)")


def command(out):
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", os.path.join(HERE, "csrc"), *srcs, "-o", out]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"libpagedkv build failed:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
