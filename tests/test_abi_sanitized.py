"""The C-ABI checks of test_abi.py again, against libkvq_san.so: the host code of the
library (argument validation, layout arithmetic, bookkeeping) built with
AddressSanitizer and UndefinedBehaviorSanitizer, loaded in a child process with
the sanitizer runtime preloaded. Needs no GPU (the device code is unchanged and
never runs)."""
import os
import subprocess
import sys

import pytest

from bit_asymmetric_kv_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_pass_under_host_sanitizers():
    if not os.path.exists(build_lib.SAN_OUT):
        pytest.skip("libkvq_san.so is built by build() / `python -m bit_asymmetric_kv_amd.build_lib --sanitize`")
    runtime = build_lib.sanitizer_runtime()
    assert runtime, "clang's shared AddressSanitizer runtime was not found"
    # the library is instrumented: it calls into both sanitizer runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", build_lib.SAN_OUT], capture_output=True, text=True,
                          check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, KVQ_LIBRARY=build_lib.SAN_OUT, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr
