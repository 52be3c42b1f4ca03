"""Host-side logic of bench.py (CPU): the one-GPU refusal, the roofline
classification and the staleness rule of the recorded GEMM traffic."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_roofline_entry_bound_and_fraction():
    # the dense step GEMM: arithmetic intensity far above the ridge point
    e = bench.roofline_entry(bench.GEMM_FLOP, bench.GEMM_MIN_BYTES, 100.0)
    assert e["bound"] == "mfma"
    assert abs(e["roofline_us"] - bench.GEMM_FLOP / (bench.FP8_PEAK_TFLOPS * 1e6)) < 1e-2
    assert abs(e["frac_roofline"] - e["roofline_us"] / 100.0) < 1e-4
    # a stream: bytes decide
    e = bench.roofline_entry(0.0, 8e6, 2.0)
    assert e["bound"] == "hbm" and abs(e["roofline_us"] - 1.0) < 1e-9 and abs(e["frac_roofline"] - 0.5) < 1e-9


def test_recorded_traffic_is_tied_to_the_gemm_source():
    """The bench reports the recorded HBM traffic only while gemm.hip hashes
    to the source the counters were taken on."""
    t = bench.GEMM_TRAFFIC
    assert t["bytes"] > bench.GEMM_MIN_BYTES and len(t["source_sha256"]) == 64
    assert "profiles/" in t["profile"]
    assert bench.source_sha256("gemm.hip") == bench.source_sha256("gemm.hip")
    assert bench.source_sha256("quant.hip") != bench.source_sha256("gemm.hip")
