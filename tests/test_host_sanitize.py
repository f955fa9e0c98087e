"""The host library's argument validation, workspace layout and parameter blocks under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU and no HIP runtime).

csrc/rs_host.cpp is compiled with g++ together with tests/host/hip_stubs.cpp (stand-ins
for the three HIP runtime calls it makes and for the kernel launchers, which check that every
pointer derived from the caller's workspace stays inside it) and the driver
tests/host/abi_sanitize_main.cpp (valid calls of every kind, and invalid calls that must
return their documented status and launch nothing).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rope_flash_attention_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC,
           "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "rs_host.cpp"), os.path.join(HOST, "hip_stubs.cpp"),
           os.path.join(HOST, "abi_sanitize_main.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " 0 failed" in r.stdout, r.stdout
