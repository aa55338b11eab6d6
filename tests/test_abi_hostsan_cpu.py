"""The C ABI's host code (argument validation, dispatch to the launchers,
error text, workspace sizing) built with AddressSanitizer and
UndefinedBehaviorSanitizer (fp8_blockwise_quantized_amd/lib/libjetfp8_hostsan.so,
made by the package build): the CPU validation tests of the boundary and of the
binding run against that build in a child process, with the sanitizer runtime
preloaded, and must pass without a sanitizer report.  No GPU: every call either
fails validation or meets the missing device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp8_blockwise_quantized_amd", "lib", "libjetfp8_hostsan.so")


def test_abi_validation_under_host_sanitizers():
    if not os.path.exists(LIB):
        pytest.skip("libjetfp8_hostsan.so is not built (python -m fp8_blockwise_quantized_amd._build)")
    from fp8_blockwise_quantized_amd import _build
    try:
        runtime = _build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=runtime, JET_LIB_PATH=LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_cpu.py", "tests/test_binding_cpu.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
