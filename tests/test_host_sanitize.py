"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C-ABI layer (argument
checks, the prefill split and decode plans, the backward chunk plan, workspace layouts) with
its kernel launches stubbed, and the CPU oracle, built with g++ / gcc for the host and driven
by tests/host_sanitize/driver.cpp (every entry point, valid and invalid arguments, every
workspace-derived buffer checked to lie inside the caller's workspace)."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "host_sanitize"))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_sanitizers(tmp_path):
    import build as hs_build

    exe = hs_build.build(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
