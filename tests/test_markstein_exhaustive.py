"""Exhaustive host check of the quantizers' element quotient (CPU).

The GPU quantizers replace the per-element IEEE division x / s by one
Markstein correction of x * RN32(1/s) (three float32 operations); a tile
with 0 < amax < 2^-90 first scales x and s by 2^64.  The C program
tests/host/markstein_check.c runs both sequences and the IEEE division on
every pair of BF16 values with |x| <= amax (521 million pairs with amax >=
2^-90, 11.2 million below) and requires equal quotients, or both at most
2^-10 (both then encode to the E4M3 zero).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "markstein_check.c")


@pytest.mark.slow
def test_markstein_quotient_equals_ieee_division_for_every_bf16_pair(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "markstein_check")
    flags = ["-O2", "-ffp-contract=off"]
    with open("/proc/cpuinfo") as f:
        if " fma " in f.read():
            flags.append("-mfma")  # hardware fused multiply-add (one rounding, like glibc's fmaf)
    build = subprocess.run([gcc, *flags, SRC, "-o", exe, "-lm"], capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "pairs 521483904" in run.stdout and "mismatches 0" in run.stdout, run.stdout
    assert "tiny pairs 11217215 equal 11217215" in run.stdout and "tiny pairs" in run.stdout, run.stdout
