"""Builds a host-only copy of the block manager and the waste simulator
with AddressSanitizer and UndefinedBehaviorSanitizer (g++, no device code),
for the CPU test that replays the manager's random-operation suites through
it.  The binding loads it in place of libpagedkv.so when the environment
variable ``PAGEDKV_HOST_ONLY_LIB`` names it (device calls are then absent).

Usage: ``python -m paged_kv_cache_354_amd.build_sanitized OUT.so``
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HOST_SOURCES = ["csrc/pa_status.cpp", "csrc/block_manager.cpp", "csrc/waste_sim.cpp"]
SANITIZERS = "address,undefined"


def gxx():
    for cand in (os.environ.get("CXX"), shutil.which("g++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("g++ not found")


def runtime_preload():
    """The sanitizer runtime a non-instrumented Python must preload to load
    the library."""
    out = subprocess.run([gxx(), "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    return out.stdout.strip()


def build(out_path, verbose=False):
    cmd = [gxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={SANITIZERS}",
           "-fno-sanitize-recover=all", "-shared", "-fPIC", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *[os.path.join(HERE, s) for s in HOST_SOURCES], "-o", out_path]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized host build failed:\n{res.stderr}")
    return out_path


if __name__ == "__main__":
    print(build(sys.argv[1], verbose=True))
