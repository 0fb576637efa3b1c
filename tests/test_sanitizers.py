"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the page pool, the scheduler and the status calls, built by g++ as a
host-only library, and the fp64 oracle, built by gcc, both instrumented, run
the CPU tests that drive them -- the pool and scheduler against their models
under hypothesis operation sequences, and the oracle's pins -- in a child
process with the ASan runtime preloaded.  Any report (heap overflow, use
after free, undefined behaviour) fails the child and this test."""

import os
import subprocess
import sys

import pytest

import oracle
from paged_kv_cache_266_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# CPU tests that exercise the instrumented code (torch is not imported in
# them: the child runs with the sanitizer runtime preloaded)
HOST_TESTS = ["tests/test_pool_lib.py", "tests/test_sched_lib.py"]
ORACLE_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_prefill.py", "tests/test_oracle_quant.py"]


def _asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(tests, env_extra, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = _asan_runtime()
    # Python itself keeps memory until exit on purpose: no leak report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *tests]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = res.stdout + res.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
    assert res.returncode == 0, text[-4000:]
    return text


@pytest.fixture(scope="module")
def runtime():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime (gcc -print-file-name=libasan.so)")
    return rt


def test_pool_and_scheduler_clean_under_asan_ubsan(runtime, tmp_path):
    lib = build.build_host(str(tmp_path / "libpagedkv_host_asan.so"), sanitize=True)
    out = _run_child(HOST_TESTS, {"PKV_HOST_LIBRARY": lib}, tmp_path)
    assert " passed" in out


def test_oracle_clean_under_asan_ubsan(runtime, tmp_path):
    lib = oracle.build(out=str(tmp_path / "liboracle_asan.so"), sanitize=True)
    out = _run_child(ORACLE_TESTS, {oracle.LIBRARY_ENV: lib, "OMP_NUM_THREADS": "4"}, tmp_path)
    assert " passed" in out


def test_sanitizer_catches_a_planted_overflow(runtime, tmp_path):
    """The harness itself: a host library with an out-of-bounds write must
    fail the child (so a clean run above means something)."""
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\n"
                   "int poke(int n) { int *a = malloc(4 * sizeof(int)); a[n] = 1; int r = a[0]; free(a); "
                   "return r; }\n")
    so = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-g", *oracle.SANITIZE_FLAGS, str(src), "-o", str(so)], check=True)
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:exitcode=87")
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).poke(4)"
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    # either sanitizer may report it first: UBSan's object-size check or ASan's redzone
    assert res.returncode in (86, 87), res.stderr[-2000:]
    assert "heap-buffer-overflow" in res.stderr or "insufficient space" in res.stderr, res.stderr[-2000:]
