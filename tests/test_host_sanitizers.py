"""The C ABI's host code (microscaling_fp4_block_mx_amd/csrc/mx_api.cpp) built
with g++ against recording launcher stubs (tests/host_sanitize/) and run
under AddressSanitizer + UndefinedBehaviorSanitizer, and separately under
ThreadSanitizer with eight threads calling at once. No kernel is built or
run: this covers validation, argument marshalling and the per-thread error
detail."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SRC = [os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc", "mx_api.cpp"),
       os.path.join(ROOT, "tests", "host_sanitize", "stubs.cpp"),
       os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")]
INC = ["/opt/rocm/include", os.path.join(ROOT, "include"),
       os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc"),
       os.path.join(ROOT, "tests", "host_sanitize")]


@pytest.mark.parametrize("flags", [["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                                   ["-fsanitize=thread"]], ids=["asan-ubsan", "tsan"])
def test_abi_host_code_under_sanitizers(tmp_path, flags):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "abi_driver")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__"] + flags
           + [f"-I{d}" for d in INC] + SRC + ["-o", exe, "-lpthread"])
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
