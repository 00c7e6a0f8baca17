"""The library's host code under sanitizers (CPU only, no device code).

* ASan + UBSan: the block manager and status code, built by
  ``build.py --sanitize`` as a host-only library, run the block-manager
  suites of test_abi.py and test_shared_prefixes.py (hypothesis against the
  oracle's allocator model) in a child process with the sanitizer runtime
  preloaded. A planted heap overflow (a caller buffer shorter than the
  capacity it claims) must be reported, which shows the runtime is active.
* TSan: tests/native/host_threads.cpp drives the launch code's caches
  (host_cache.h) from 16 threads and independent block managers from 8,
  checking the thread-local error strings; a planted unsynchronised counter
  must be reported.
"""
import os
import shutil
import subprocess
import sys

import pytest

from paged_kv_cache_49_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")

BM_TESTS = ("status_strings or block_manager or prefix_cache or usage or swapped or worked_examples or "
            "parallel_sampling or bad_granule or random_histories")


def _runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()


def _asan_env(lib: str) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=_runtime("libasan.so"), PA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


@pytest.fixture(scope="module")
def asan_lib():
    return B.build_sanitized("asan")


def test_block_manager_suites_under_asan_ubsan(asan_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-k", BM_TESTS,
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_shared_prefixes.py")],
                       cwd=ROOT, env=_asan_env(asan_lib), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and "13 passed" in out, out[-2000:]


def test_asan_reports_a_planted_overflow(asan_lib):
    """pa_bm_free_stack told a capacity of 40 for an 8-byte malloc buffer."""
    code = (
        "import ctypes\n"
        "from paged_kv_cache_49_amd import _lib\n"
        "lib = _lib.lib(); libc = ctypes.CDLL(None)\n"
        "libc.malloc.restype = ctypes.c_void_p\n"
        "bm = ctypes.c_void_p(); assert lib.pa_bm_create(40, 16, None, ctypes.byref(bm)) == 0\n"
        "buf = libc.malloc(8); n = ctypes.c_int32()\n"
        "lib.pa_bm_free_stack(bm, buf, 40, ctypes.byref(n))\n"
        "print('not reported')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_asan_env(asan_lib), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-3000:]


@pytest.fixture(scope="module")
def tsan_driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("tsan") / "host_threads")
    cmd = ["g++", *B.sanitize_flags("tsan"), os.path.join(NATIVE, "host_threads.cpp"),
           *[os.path.join(B.CSRC, f) for f in B.HOST_SOURCES], "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _tsan_env() -> dict:
    env = dict(os.environ)
    env["TSAN_OPTIONS"] = "halt_on_error=1:exitcode=66"
    return env


def test_host_caches_and_managers_under_tsan(tsan_driver):
    r = subprocess.run([tsan_driver], env=_tsan_env(), capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ThreadSanitizer" not in out, out[-4000:]
    assert "caches: 0 bad" in out and "managers: 0 bad" in out, out


def test_tsan_reports_a_planted_race(tsan_driver):
    r = subprocess.run([tsan_driver, "--planted-race"], env=_tsan_env(), capture_output=True, text=True, timeout=300)
    assert r.returncode == 66 and "data race" in r.stderr, (r.stdout + r.stderr)[-3000:]
