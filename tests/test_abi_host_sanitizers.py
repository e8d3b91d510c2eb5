"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host layer (argument validation, workspace arithmetic, the device
check, status strings) is rebuilt without device code and with both sanitizers,
then every case of test_abi_cpu.py runs against it in a child process with the
shared sanitizer runtime preloaded. Any report aborts the child (no recovery),
so a clean exit means no memory error and no undefined behaviour on those paths.
"""

import os
import shutil
import subprocess
import sys

import pytest

from ragged_grouped_gemm_histogram_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def _toolchain_ok() -> bool:
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return os.path.exists(B.clangxx()) and os.path.exists(B.sanitizer_runtime())


@pytest.mark.skipif(not shutil.which("hipcc") and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_abi_host_code_is_clean_under_asan_and_ubsan():
    if not _toolchain_ok():
        pytest.skip("sanitizer runtime not found")
    lib = B.build_host_sanitized()
    env = dict(os.environ)
    env.update({
        "MOE_TEST_LIB": lib,
        "LD_PRELOAD": B.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_cpu.py"), "-q", "-s",
                          "-p", "no:cacheprovider", "-p", "no:xdist"],
                         env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    tail = res.stdout[-4000:]
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stdout and "ERROR: AddressSanitizer" not in res.stdout, tail
