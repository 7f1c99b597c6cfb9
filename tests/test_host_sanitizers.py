"""The host block manager and the waste simulator under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

A host-only copy of ``block_manager.cpp`` and ``waste_sim.cpp`` is built with
``-fsanitize=address,undefined -fno-sanitize-recover=all`` and the manager's
CPU suites (the golden traces, the hypothesis and seeded random-operation
runs against the oracle's model, the waste simulator against its oracle)
are replayed through it in a child process: any heap overflow, use after
free, double free or undefined behaviour aborts the child and fails this
test.  Leak checking is off (the interpreter itself holds memory at exit).
"""

import os
import subprocess
import sys

import pytest

from paged_kv_cache_354_amd import HOST_ONLY_ENV
from paged_kv_cache_354_amd import build_sanitized as BS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_block_manager.py", "tests/test_oracle_manager.py", "tests/test_waste.py"]


def test_manager_suites_under_asan_ubsan(tmp_path):
    try:
        lib = BS.build(str(tmp_path / "libpagedkv_host_asan.so"))
        preload = BS.runtime_preload()
    except (RuntimeError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    env = dict(os.environ)
    env[HOST_ONLY_ENV] = lib
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *SUITES],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout[-3000:] + "\n" + res.stderr[-3000:])
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
    assert "runtime error" not in res.stderr, tail

    # the suites ran on the sanitized host-only build, not on libpagedkv.so
    probe = ("import paged_kv_cache_354_amd as p; l = p.load(); "
             f"assert l._name == {lib!r}, l._name; assert not hasattr(l, 'pa_decode'); print('host-only ok')")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0 and "host-only ok" in res.stdout, res.stderr[-2000:]


def test_sanitizer_setup_catches_a_planted_overflow(tmp_path):
    """The same flags and preload abort a child on a one-past-the-end heap
    write in a library it loads (so a clean run above means something)."""
    src = tmp_path / "planted.cpp"
    src.write_text('extern "C" int planted(int n) { int *a = new int[n]; a[n] = 1; int r = a[0]; '
                   'delete[] a; return r; }\n')
    so = tmp_path / "libplanted.so"
    try:
        subprocess.run([BS.gxx(), "-O1", "-g", f"-fsanitize={BS.SANITIZERS}", "-fno-sanitize-recover=all",
                        "-shared", "-fPIC", str(src), "-o", str(so)], check=True, capture_output=True)
        preload = BS.runtime_preload()
    except (RuntimeError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).planted(4)"
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]
