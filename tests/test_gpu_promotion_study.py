"""Promotion-interval study on the weight-gradient workload, GPU part: the
library's accumulation forms against the exact value (GPU + oracle).

dW = dY^T X over 16384 tokens (dY 16384 x 2048, X 16384 x 7168, BF16
~N(0,1), 128-token x 1-feature tiles).  On the seeded 256 x 256 sample of
dW (65,536 elements, tests/promotion_sample.py) the error against the exact
value is reported for the GPU path:

  * libfp8q wgrad, partial sums over 128 tokens promoted to FP32 with the
    tile scales, the partials formed at float32 grade (default) and inside
    the FP8 matrix core (acc="fp8_mfma");
  * with power-of-two scales: the same two, the matrix core applying the
    scales and keeping the whole sum (acc="fp8_mfma_scaled", no promotion),
    and the BF16 matrix core keeping the whole sum in float32 with the scales
    applied exactly in the operands (acc="fp32_pow2", no promotion).

The hardware model of the FP8 unit (tests/fp8_unit_model.py) is set next to
the measured FP8-unit form on a 64 x 64 corner of the sample.  The emulated
accumulators (float32 and W-bit fixed point, promoted every 128 products and
not at all) run on the same 65,536 elements on the CPU
(tests/test_promotion_emulators.py).

The pages: limited accumulation width inside the matrix unit
(why-be.co.kr wr_id=35533 ¶4), fixed-point alignment by right shifts
(tmdrlife.com wr_id=13334 ¶2), promotion every 128 elements as the remedy
(jp-study.kr doc 258368 ¶3).  Errors are |value - exact| / sum_k |a_k b_k|
(the normalisation of the GEMM tolerance).  The report is printed and, when
FP8Q_STUDY_OUT names a file, written there as JSON.
"""

import json
import os

import numpy as np
import pytest

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from gpu_util import assert_codes_equal, assert_scales_equal, dev_bf16, host, host_codes, need_gpu, say
from oracle import quantize as Q
import fp8_unit_model as unit
import promotion_sample as P

pytestmark = pytest.mark.gpu

CORNER = 64  # rows and columns of the sample's corner compared with the FP8-unit model


def test_promotion_study():
    need_gpu()
    d = synth.wgrad()
    t, nout = d["dy"].shape
    kin = d["x"].shape[1]
    report = {"workload": f"dW {nout}x{kin}, T={t}, sample {P.SIDE}x{P.SIDE} = {P.SIDE * P.SIDE} elements"}
    for mode, qm in (("free", Q.FREE), ("pow2", Q.POW2)):
        say(f"[study] GPU quantization + wgrad {nout}x{kin} over {t} tokens ({mode} scales)")
        dyq, dysq = fp8q.quantize_act(dev_bf16(d["dy"]), tile_axis="token_t", scale_mode=mode)
        xq, xsq = fp8q.quantize_act(dev_bf16(d["x"]), tile_axis="token_t", scale_mode=mode)
        ops = P.operands(d, qm)
        rsel, csel = ops["rsel"], ops["csel"]
        # the GPU operands of the sampled features are the oracle's, bit for bit
        assert_codes_equal(host_codes(dyq)[rsel], ops["dyc"], f"dY codes ({mode})")
        assert_codes_equal(host_codes(xq)[csel], ops["xc"], f"X codes ({mode})")
        assert_scales_equal(host(dysq)[rsel], ops["dys"], f"dY scales ({mode})")
        assert_scales_equal(host(xsq)[csel], ops["xs"], f"X scales ({mode})")
        forms = (("gpu_interval_128", "fp32"), ("gpu_fp8_mfma_interval_128", "fp8_mfma"))
        if mode == "pow2":
            forms += (("gpu_fp8_mfma_scaled_no_promotion", "fp8_mfma_scaled"),
                      ("gpu_fp32_grade_no_promotion", "fp32_pow2"))
        prefix = "" if mode == "free" else "pow2_"
        for name, acc in forms:
            got = host(fp8q.wgrad(dyq, dysq, xq, xsq, acc=acc)).astype(np.float64)[np.ix_(rsel, csel)]
            report[prefix + name] = P.stats(got, ops["exact"], ops["s"])
            if mode == "free" and acc == "fp8_mfma":
                # the hardware model of the FP8 unit beside the measurement,
                # on the sample's 64 x 64 corner
                ri = np.repeat(np.arange(CORNER), CORNER)
                ci = np.tile(np.arange(CORNER), CORNER)
                model, _, _ = unit.gemm_at_mfma(ops["dyc"], ops["dys"], ops["xc"], ops["xs"], ri, ci,
                                                w_block_rows=False)
                ex, s = ops["exact"][:CORNER, :CORNER], ops["s"][:CORNER, :CORNER]
                report["gpu_fp8_mfma_interval_128_corner"] = P.stats(got[:CORNER, :CORNER], ex, s)
                report["model_fp8_mfma_interval_128_corner"] = P.stats(model, ex, s)
        del dyq, dysq, xq, xsq

    say(json.dumps(report, indent=1))
    out = os.environ.get("FP8Q_STUDY_OUT")
    if out:
        with open(out, "w") as f:
            json.dump(report, f, indent=1)

    assert report["gpu_interval_128"]["within_tolerance"] == 1.0
    assert report["pow2_gpu_interval_128"]["within_tolerance"] == 1.0
    # float32 accumulation of the whole sum, scales applied exactly in the
    # operands (no promotion step): float32 grade too
    assert report["pow2_gpu_fp32_grade_no_promotion"]["within_tolerance"] == 1.0
