"""Promotion-interval study on the weight-gradient workload, CPU part: the
accumulation emulators (oracle.accum) on the seeded 256 x 256 sample of dW
(65,536 elements, tests/promotion_sample.py; the GPU part,
tests/test_gpu_promotion_study.py, measures the library's forms on the same
elements).

dW = dY^T X over 16384 tokens (dY 16384 x 2048, X 16384 x 7168, BF16
~N(0,1), 128-token x 1-feature tiles, free scales, quantized by the oracle).
For every sampled element the 16384 dequantized products (a sa)(b sb) are
summed by a float32 accumulator and by W-bit fixed-point accumulators
aligned to the running maximum exponent (W = 13, 14, 16, 20), each promoted
to a float32 register every 128 products and not at all (one accumulator
over all 16384 products).  Errors are |value - exact| / sum_k |a_k b_k|.

The pages: limited accumulation width inside the matrix unit
(why-be.co.kr wr_id=35533 ¶4), fixed-point alignment by right shifts
(tmdrlife.com wr_id=13334 ¶2), promotion every 128 elements as the remedy
(jp-study.kr doc 258368 ¶3).  The report is printed and, when
FP8Q_EMULATOR_OUT names a file, written there as JSON.
"""

import json
import os
import sys

import numpy as np
import pytest

import synth
from tests import promotion_sample as P


@pytest.mark.slow
def test_promotion_emulators():
    d = synth.wgrad()
    t = d["dy"].shape[0]
    ops = P.operands(d)
    del d
    configs = P.emulator_configs(t)
    sums = P.emulate(ops, configs, workers=max(1, min(8, len(os.sched_getaffinity(0)))))
    report = {"workload": f"dW 2048x7168, T={t}, sample {P.SIDE}x{P.SIDE} = {P.SIDE * P.SIDE} elements"}
    for name, _, _ in configs:
        report[f"emulated_{name}"] = P.stats(sums[name], ops["exact"], ops["s"])
    print(json.dumps(report, indent=1), file=sys.stderr)
    out = os.environ.get("FP8Q_EMULATOR_OUT")
    if out:
        with open(out, "w") as f:
            json.dump(report, f, indent=1)

    # float32 partials promoted every 128: inside the GEMM tolerance
    assert report["emulated_fp32_interval_128"]["within_tolerance"] == 1.0
    # promotion is what keeps a narrow accumulator usable: at every width the
    # promoted sum is more accurate than the unpromoted one, and a wider
    # accumulator is more accurate than a narrower one
    for w in P.WIDTHS:
        assert (report[f"emulated_fixed{w}_interval_128"]["mean_err_over_S"]
                < report[f"emulated_fixed{w}_no_promotion"]["mean_err_over_S"])
    for lo_w, hi_w in zip(P.WIDTHS, P.WIDTHS[1:]):
        assert (report[f"emulated_fixed{hi_w}_interval_128"]["mean_err_over_S"]
                < report[f"emulated_fixed{lo_w}_interval_128"]["mean_err_over_S"])
