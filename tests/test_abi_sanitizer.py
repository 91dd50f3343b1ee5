"""The C ABI's host code (argument validation in fa_api.cpp, launch planning in
fa_plan.cpp) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every entry point by tests/abi_host/abi_checks.cpp, with stub
launchers in place of the kernels.  Host only: nothing here needs a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_tiled_03_amd", "csrc")


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path / "abi_checks")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Werror", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(ROOT, "tests", "abi_host", "abi_checks.cpp"),
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stdout
    assert "0 failed" in r.stdout
