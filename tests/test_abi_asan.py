"""The C ABI's host-side argument validation under AddressSanitizer.

The CPU tests of the ABI (test_abi_cpu.py) run again in a child process against
libsvdq_asan.so, whose C-ABI source has its host code instrumented, with the compiler's
ASan runtime preloaded.  An invalid host memory access in the validation or the size
queries aborts the child with an ASan report, which fails this test."""

import os
import subprocess
import sys

import pytest

from w4a4_rank_corrected_linear_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = ("import ctypes, sys\n"
         "import w4a4_rank_corrected_linear_amd._lib as L\n"
         "L.lib()\n"
         "ctypes.CDLL(None).__asan_init\n"   # the runtime is in the process
         "print('asan-ok', L.LIB_PATH)\n")


def test_abi_validation_under_host_asan():
    try:
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_asan()
    with open(lib, "rb") as f:
        assert b"__asan_report_load" in f.read(), "the library's host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, SVDQ_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    probe = subprocess.run([sys.executable, "-c", PROBE], env=env, cwd=ROOT,
                           capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and "asan-ok" in probe.stdout, probe.stderr[-4000:]
    assert lib in probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout
