"""The C ABI's host-side argument checks under AddressSanitizer and UBSan
(CPU only). tests/asan/host_checks.cpp links io_aware_tiled_09_amd/csrc/
fa_api.cpp against stub launchers and drives every entry point through valid
calls and each kind of refused call on fake device addresses; any
out-of-bounds access, leak or undefined behaviour in the checks aborts the
run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_argument_checks_under_asan(tmp_path):
    exe = tmp_path / "host_checks"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "asan", "host_checks.cpp"),
           os.path.join(ROOT, "io_aware_tiled_09_amd", "csrc", "fa_api.cpp"),
           os.path.join(ROOT, "io_aware_tiled_09_amd", "csrc", "fa_plan.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok: 6 launches reached the stubs" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr
