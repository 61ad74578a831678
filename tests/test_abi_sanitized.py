"""The C ABI's host code (fa_api.cpp) built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer, linked with host-only launcher stubs, and
driven by tests/abi_host/abi_host_check.cpp: argument rejection, the launch
parameters of valid calls, NULL pointers of empty tensors and the opt-in
FA_DEBUG_VALIDATE check of device index arrays. Runs on the CPU; no GPU code
is built."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "abi_host")
CSRC = os.path.join(ROOT, "io_aware_exact_flashattention_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    srcs = [os.path.join(CSRC, "fa_api.cpp"), os.path.join(HOST, "hip_stub.cpp"),
            os.path.join(HOST, "abi_host_check.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", HOST, *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("FA_DEBUG_VALIDATE", None)
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "checks passed" in r.stdout
