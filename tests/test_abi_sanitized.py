"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libmoe_san.so is the library's host code alone (no device code), compiled
with ASan + UBSan (routing_grouped_gemm_gemv_amd.build.build_sanitized).  The
CPU ABI tests (argument validation, error strings, workspace sizes, every
error path that returns before a device is touched) run against it in a
child process that preloads the ASan runtime; any report of either
sanitizer fails the run.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_abi_tests_under_asan_and_ubsan():
    from routing_grouped_gemm_gemv_amd import build as bld

    lib = bld.build_sanitized()
    env = dict(os.environ)
    env.update({
        "MOE_LIB": lib,
        "LD_PRELOAD": bld.asan_runtime(),
        # the interpreter and torch are not instrumented: leaks and the
        # interceptors' view of their allocations are not this library's
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
        "PYTHONPATH": ROOT,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
