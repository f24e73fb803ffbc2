"""The library's host-only code (host.cpp and sched.cpp) built with the host
compiler alone under AddressSanitizer and UndefinedBehaviorSanitizer, and
driven through its C ABI by tests/sanitize_driver.cpp: valid inputs, every
error path and seeded random tables, pools, request sets and rank
allocations.  Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tenant_composite_lora_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "sched.cpp"),
           os.path.join(ROOT, "tests", "sanitize_driver.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    if "LeakSanitizer does not work under ptrace" in out or "LeakSanitizer has encountered a fatal error" in out:
        env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1:detect_leaks=0"
        r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
        out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out
