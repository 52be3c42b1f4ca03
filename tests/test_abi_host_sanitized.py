"""The host code of the C ABI (argument checks, the device check and its
cache, the hand-over of every argument to the kernel launchers) built for
the CPU with AddressSanitizer and UndefinedBehaviorSanitizer, with the
launchers and the two HIP runtime queries stubbed out
(tests/host_abi_check.cpp), and run through every entry point."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_fp8_fp8q_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


def test_host_abi_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "host_abi_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fp8q_api.cpp"), os.path.join(ROOT, "tests", "host_abi_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host ABI checks passed" in run.stdout
