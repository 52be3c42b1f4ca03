"""Promotion-interval study on the weight-gradient workload (GPU + oracle).

dW = dY^T X over 16384 tokens (dY 16384 x 2048, X 16384 x 7168, BF16
~N(0,1), 128-token x 1-feature tiles).  For a seeded sample of dW elements
(64 rows x 64 columns), the error against the exact value is reported for

  * the GPU path (libfp8q wgrad: partial sums over 128 tokens, promoted to
    FP32 with the tile scales) -- measured, with the partials formed at
    float32 grade (default) and inside the FP8 matrix core (acc="fp8_mfma"),
    next to the hardware model of that unit (tests/fp8_unit_model.py); and, with power-of-two scales,
    the matrix core applying the scales and keeping the whole sum
    (acc="fp8_mfma_scaled", no promotion) and the BF16 matrix core
    keeping the whole sum in float32 with the scales applied exactly in the
    operands (acc="fp32_pow2", no promotion) next to the promoted forms;
  * emulated accumulators (oracle.accum): a float32 accumulator and a W-bit
    fixed-point accumulator aligned to the running maximum exponent, each
    with promotion every 128 products and with no promotion at all (one
    accumulator over all 16384 products).

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
from gpu_util import (assert_codes_equal, assert_scales_equal, dev_bf16, host, host_codes, need_gpu,
                      say)
from oracle import accum, gemm as G, quantize as Q
import fp8_unit_model as unit

pytestmark = pytest.mark.gpu

WIDTHS = (13, 14, 16, 20)
SAMPLE = 64  # rows and columns of dW in the sample (SAMPLE^2 elements)


def _stats(value, exact, s):
    err = np.abs(np.asarray(value, np.float64) - exact)
    rel = err / s
    tol_ok = err <= G.tolerance(s)
    nz = exact != 0
    return {"max_err_over_S": float(rel.max()), "mean_err_over_S": float(rel.mean()),
            "median_err_over_abs": float(np.median(err[nz] / np.abs(exact[nz]))),
            "within_tolerance": float(tol_ok.mean())}


def test_promotion_study():
    need_gpu()
    d = synth.wgrad()
    t, nout = d["dy"].shape
    kin = d["x"].shape[1]
    say(f"[study] GPU quantization + wgrad {nout}x{kin} over {t} tokens")
    dyq, dysq = fp8q.quantize_act(dev_bf16(d["dy"]), tile_axis="token_t")
    xq, xsq = fp8q.quantize_act(dev_bf16(d["x"]), tile_axis="token_t")
    dw = host(fp8q.wgrad(dyq, dysq, xq, xsq)).astype(np.float64)
    dw_mfma = host(fp8q.wgrad(dyq, dysq, xq, xsq, acc="fp8_mfma")).astype(np.float64)

    rng = np.random.default_rng(2024)
    rsel = np.sort(rng.choice(nout, SAMPLE, replace=False))
    csel = np.sort(rng.choice(kin, SAMPLE, replace=False))
    say("[study] oracle quantization of the sampled features")
    dyc, dys = Q.quantize_token_t(d["dy"][:, rsel])
    xc, xs = Q.quantize_token_t(d["x"][:, csel])
    # the GPU operands of the sampled features are the oracle's, bit for bit
    assert_codes_equal(host_codes(dyq)[rsel], dyc, "dY codes")
    assert_codes_equal(host_codes(xq)[csel], xc, "X codes")
    assert_scales_equal(host(dysq)[rsel], dys, "dY scales")
    assert_scales_equal(host(xsq)[csel], xs, "X scales")
    ri = np.repeat(np.arange(SAMPLE), SAMPLE)
    ci = np.tile(np.arange(SAMPLE), SAMPLE)
    rows, cols = rsel[ri], csel[ci]
    exact, s = G.gemm_at(dyc, dys, xc, xs, ri, ci, w_block_rows=False)

    report = {"workload": f"dW {nout}x{kin}, T={t}, sample {rows.size} elements",
              "gpu_interval_128": _stats(dw[rows, cols], exact, s),
              # partials formed inside the FP8 matrix core (limited-width
              # alignment), promoted every 128 as above
              "gpu_fp8_mfma_interval_128": _stats(dw_mfma[rows, cols], exact, s)}
    model, _, _ = unit.gemm_at_mfma(dyc, dys, xc, xs, ri, ci, w_block_rows=False)
    report["emulated_fp8_mfma_interval_128"] = _stats(model, exact, s)
    say("[study] emulators")
    terms = accum.dequantized_products(dyc[ri], dys[ri], xc[ci], xs[ci])
    report["emulated_fp32_interval_128"] = _stats(accum.accumulate(terms, 128), exact, s)
    report["emulated_fp32_no_promotion"] = _stats(accum.accumulate(terms, t), exact, s)
    for w in WIDTHS:
        report[f"emulated_fixed{w}_interval_128"] = _stats(accum.accumulate(terms, 128, w), exact, s)
        report[f"emulated_fixed{w}_no_promotion"] = _stats(accum.accumulate(terms, t, w), exact, s)

    # the same workload with power-of-two scales, where the matrix core can
    # apply the scales itself and keep the whole sum: promotion every 128 vs
    # none, both measured on the GPU
    say("[study] power-of-two scales: promoted vs unpromoted on the matrix core")
    dyq2, dys2 = fp8q.quantize_act(dev_bf16(d["dy"]), tile_axis="token_t", scale_mode="pow2")
    xq2, xs2 = fp8q.quantize_act(dev_bf16(d["x"]), tile_axis="token_t", scale_mode="pow2")
    dyc2, dysc2 = Q.quantize_token_t(d["dy"][:, rsel], Q.POW2)
    xc2, xsc2 = Q.quantize_token_t(d["x"][:, csel], Q.POW2)
    assert_codes_equal(host_codes(dyq2)[rsel], dyc2, "dY codes (pow2)")
    assert_codes_equal(host_codes(xq2)[csel], xc2, "X codes (pow2)")
    exact2, s2 = G.gemm_at(dyc2, dysc2, xc2, xsc2, ri, ci, w_block_rows=False)
    for name, acc in (("fp32_interval_128", "fp32"), ("fp8_mfma_interval_128", "fp8_mfma"),
                      ("fp8_mfma_scaled_no_promotion", "fp8_mfma_scaled"),
                      ("fp32_grade_no_promotion", "fp32_pow2")):
        got = host(fp8q.wgrad(dyq2, dys2, xq2, xs2, acc=acc)).astype(np.float64)
        report[f"pow2_gpu_{name}"] = _stats(got[rows, cols], exact2, s2)

    say(json.dumps(report, indent=1))
    out = os.environ.get("FP8Q_STUDY_OUT")
    if out:
        with open(out, "w") as f:
            json.dump(report, f, indent=1)

    assert report["gpu_interval_128"]["within_tolerance"] == 1.0
    assert report["emulated_fp32_interval_128"]["within_tolerance"] == 1.0
    assert report["pow2_gpu_fp32_interval_128"]["within_tolerance"] == 1.0
    # float32 accumulation of the whole sum, scales applied exactly in the
    # operands (no promotion step): float32 grade too
    assert report["pow2_gpu_fp32_grade_no_promotion"]["within_tolerance"] == 1.0
    # promotion is what keeps a narrow accumulator usable: at every width the
    # promoted sum is more accurate than the unpromoted one
    for w in WIDTHS:
        assert (report[f"emulated_fixed{w}_interval_128"]["mean_err_over_S"]
                < report[f"emulated_fixed{w}_no_promotion"]["mean_err_over_S"])
