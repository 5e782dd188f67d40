"""CPU test: the argument-checking paths of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer.

Builds libmoe_san.so (the layer's sources with host-side ASan + UBSan; device
code as usual) and runs tests/test_abi.py in a child process that preloads the
sanitizer runtime and loads that build through MOE_LIBRARY. Every call there is
rejected on the host before any HIP call, so no GPU is needed; a sanitizer
report aborts the child and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the sanitizer library")
def test_abi_checks_under_address_and_undefined_sanitizers():
    sys.path.insert(0, ROOT)
    from sparse_mixture_experts_fp32_amd import build as b
    lib = b.build_sanitized(verbose=False)
    runtime = b.sanitizer_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, MOE_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import ctypes, sys; "
            "assert hasattr(ctypes.CDLL(None), '__asan_init'), 'sanitizer runtime not loaded'; "
            "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
