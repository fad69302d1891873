"""The host layer (include/pkv.h entry points, allocator, prefix cache,
slot mapping, precondition checks, workspace sizing) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU
(tests/sanitize/driver.cpp against the stubs in tests/sanitize/stubs.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_layer_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "pkv_host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "paged_kv_attention_06_amd", "csrc"),
           os.path.join(ROOT, "paged_kv_attention_06_amd", "csrc", "pkv_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("PKV_DEBUG_VALIDATE", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host layer under ASan/UBSan: ok" in r.stdout
