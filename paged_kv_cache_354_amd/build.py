"""Builds libpagedkv.so (HIP kernels + C ABI + host block manager) for gfx950.

Usage: ``python -m paged_kv_cache_354_amd.build`` (also called by
``__graft_entry__.build``).  The library is written next to this file.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedkv.so")
SOURCES = [
    "csrc/pa_status.cpp",
    "csrc/block_manager.cpp",
    "csrc/waste_sim.cpp",
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


COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extra flags.  The prefill kernel keeps its matrix-core
# accumulators in ordinary VGPRs: its online-softmax rescale and its use of
# the scores would otherwise copy them out of and back into AGPRs.
EXTRA_FLAGS = {
    "csrc/pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def compile_command(src, obj):
    return [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", os.path.join(HERE, "csrc"),
            "-c", os.path.join(HERE, src), "-o", obj]


def link_command(objs, out):
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"libpagedkv build failed:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False):
    """Compile every source to an object (in parallel, in a temporary
    directory), link libpagedkv.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="pagedkv_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            list(ex.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
        tmp = LIB + ".tmp"
        _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
