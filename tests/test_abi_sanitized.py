"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (validation, error codes, workspace sizes) and plan.cpp (split plans) are built with
g++ and -fsanitize=address,undefined into a host-only library whose kernel launchers are stubs
(tests/asan/launch_stub.cpp), and the ABI validation tests of test_abi_cpu.py run against it in
a child interpreter with the ASan runtime preloaded.  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_flash_attn_fwd_amd", "csrc")


def _gxx():
    return shutil.which("g++")


@pytest.mark.skipif(_gxx() is None, reason="g++ not available")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    gxx = _gxx()
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not available")
    lib = str(tmp_path / "libattn_host_sanitized.so")
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-shared", "-fPIC", *sanitize, "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stub.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ATTN_ABI_TEST_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
