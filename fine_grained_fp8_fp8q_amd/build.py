"""Builds libfp8q.so (gfx950 only) in place with hipcc, and the bench's
streaming reference libfp8q_streamref.so.

    python -m fine_grained_fp8_fp8q_amd.build

Every call recompiles all sources.  Objects go to <repo>/_build/, the shared
library next to this file.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8q.so")
# the bench's plain streaming kernel (a measuring stick, not part of libfp8q)
STREAMREF_LIB = os.path.join(PKG, "libfp8q_streamref.so")

SOURCES = ["quant.hip", "gemm.hip", "gemm_small.hip", "moe.hip", "fp8q_api.cpp"]

# -ffp-contract=off: every fused multiply-add in the kernels is written out
# explicitly (the quotient correction and the scale fold depend on it).
# -packed-fp32-ops: no packed FP32 VALU instructions are generated.
# -amdgpu-mfma-vgpr-form: MFMA results land in VGPRs, where the FP32 scale
# fold reads them, instead of AGPRs that would need a copy per element.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8q.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host launch stub the compiler failed to
    # emit shows up here instead of when the library is loaded
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    tmp = STREAMREF_LIB + ".tmp"
    _run([cc, *COMMON, "-shared", "-Wl,--no-undefined", os.path.join(CSRC, "stream_ref.hip"), "-o", tmp], verbose)
    os.replace(tmp, STREAMREF_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
