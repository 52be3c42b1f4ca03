"""Exhaustive host check of the quantizers' tile scale and its reciprocal (CPU).

The GPU quantizers form s = RN32(amax / 448) with one Markstein correction of
amax * RN32(1/448), and RN32(1 / s) (or of s * 2^64 for a tile with
0 < amax < 2^-90) with one Newton step from the hardware reciprocal.
tests/host/scale_reciprocal_check.c runs both on every nonzero finite BF16
amax (32,639 values) and requires the scale to equal the IEEE quotient bit
for bit and the reciprocal to equal the IEEE reciprocal from every starting
value within 2 ulps of it.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "scale_reciprocal_check.c")


def test_scale_and_reciprocal_equal_ieee_for_every_bf16_amax(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "scale_reciprocal_check")
    flags = ["-O2", "-ffp-contract=off"]
    with open("/proc/cpuinfo") as f:
        if " fma " in f.read():
            flags.append("-mfma")  # hardware fused multiply-add (one rounding, like glibc's fmaf)
    build = subprocess.run([gcc, *flags, SRC, "-o", exe, "-lm"], capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "amax values 32639 scale mismatches 0 reciprocal starts 163195 mismatches 0" in run.stdout, run.stdout
