"""The C ABI's CPU tests (tests/test_abi.py) run again against a build whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer: argument
checks, workspace sizing and carving, and the plain C caller.  No GPU is
involved; device code is built exactly as in the product library."""

import os
import subprocess
import sys

from sparse_moe_layer_wave_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers():
    lib = build.build(verbose=False, sanitize=True)
    # the host code really is instrumented: it calls into both runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                          check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, HY3MOE_LIBRARY=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
