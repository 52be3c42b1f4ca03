"""The opt-in FP8-unit accumulation forms against the oracle at the stated
tolerance |gpu - oracle| <= 1e-5 * S + 1e-6 (no hardware model involved).

FP8Q_ACC_FP8_MFMA forms each 128-element partial inside the FP8 matrix core
and promotes it to FP32 with the scales (tmdrlife.com wr_id=13334 ¶3,
jp-study.kr doc 258368 ¶3); FP8Q_ACC_FP8_MFMA_SCALED (power-of-two scales)
hands the scales to the matrix core and keeps the whole sum there (the
pages' "MMA with group scaling", tmdrlife.com wr_id=13334 ¶3).  The unit
aligns the products of each group of 8 to the group's largest one (the
limited-width accumulation of why-be.co.kr wr_id=35533 ¶4), so whether these
forms meet the tolerance depends on the operands' spread inside a group:

* the weight-gradient workload (dY 16384 x 2048, X 16384 x 7168, ~N(0,1),
  128-token tiles; free and power-of-two scales) meets it: asserted here on
  sampled outputs and on two whole 256 x 224 output tiles;
* so does the activation gradient of the up-projection (dY 4096 x 4096
  ~N(0,1) in 1x128 tiles times W 4096 x 7168 ~N(0,0.02)): asserted on
  sampled outputs and on two whole 256 x 224 output tiles;
* the workloads with outliers (tiny linear: 0.5% of A x50; dense
  up-projection and MoE: 0.1% x100) do not: their fractions within tolerance
  are measured and reported (printed, and written as JSON when
  FP8Q_UNIT_REPORT names a file), not asserted.

The float32-grade default form meets the tolerance on every workload (the
other GPU GEMM tests).
"""

import json
import os

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from oracle import gemm as G, quantize as Q
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, dev, dev_bf16, host, host_bf16_bits,
                            host_codes, moe_operands, need_gpu, say)

pytestmark = pytest.mark.gpu

_WGRAD = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _wgrad_operands(mode):
    """GPU token-axis quantization of the full Wgrad workload, with the
    features that the checks below read compared bit for bit with the
    oracle's quantization of the same columns."""
    if mode not in _WGRAD:
        if "bf16" not in _WGRAD:
            _WGRAD["bf16"] = synth.wgrad()
        d = _WGRAD["bf16"]
        t, nout = d["dy"].shape
        kin = d["x"].shape[1]
        say(f"[fp8-unit] wgrad operands {nout}x{kin} over {t} tokens, {mode} scales")
        dyq, dys = fp8q.quantize_act(dev_bf16(d["dy"]), tile_axis="token_t", scale_mode=mode)
        xq, xs = fp8q.quantize_act(dev_bf16(d["x"]), tile_axis="token_t", scale_mode=mode)
        rng = np.random.default_rng(77)
        # rows/columns: the sample plus two whole 256 x 224 output tiles (the
        # first tile and the last full-width one)
        rsel = np.unique(np.concatenate([rng.choice(nout, 48, replace=False), np.arange(256),
                                         np.arange(nout - 256, nout)]))
        csel = np.unique(np.concatenate([rng.choice(kin, 48, replace=False), np.arange(224),
                                         np.arange(kin - 224, kin)]))
        qm = Q.POW2 if mode == "pow2" else Q.FREE
        dyc, dysc = Q.quantize_token_t(d["dy"][:, rsel], qm)
        xc, xsc = Q.quantize_token_t(d["x"][:, csel], qm)
        assert_codes_equal(host_codes(dyq)[rsel], dyc, "dY codes")
        assert_scales_equal(host(dys)[rsel], dysc, "dY scales")
        assert_codes_equal(host_codes(xq)[csel], xc, "X codes")
        assert_scales_equal(host(xs)[csel], xsc, "X scales")
        _WGRAD[mode] = (dyq, dys, xq, xs, rsel, csel, (dyc, dysc, xc, xsc))
    return _WGRAD[mode]


@pytest.mark.parametrize("mode,acc", [("free", "fp8_mfma"), ("pow2", "fp8_mfma"), ("pow2", "fp8_mfma_scaled")])
def test_fp8_unit_forms_meet_tolerance_on_wgrad(mode, acc):
    dyq, dys, xq, xs, rsel, csel, ops = _wgrad_operands(mode)
    nout, kin = dyq.shape[0], xq.shape[0]
    say(f"[fp8-unit] wgrad {nout}x{kin} acc={acc} scales={mode}")
    dw = host(fp8q.wgrad(dyq, dys, xq, xs, acc=acc)).astype(np.float64)
    # whole tiles: the oracle's wgrad on the selected features, every element
    # of the first and the last-but-ragged 256 x 224 tile
    ref, s = G.wgrad(*ops)
    got = dw[np.ix_(rsel, csel)]
    ok = G.accept_f32(got, ref, s)
    assert ok.all(), (f"wgrad {acc} ({mode}): {int((~ok).sum())} of {ok.size} outside 1e-5*S+1e-6; "
                      f"max err/S {float((np.abs(got - ref) / s).max()):.3g}")


_DGRAD = {}


@pytest.mark.parametrize("mode,acc", [("free", "fp8_mfma"), ("pow2", "fp8_mfma"), ("pow2", "fp8_mfma_scaled")])
def test_fp8_unit_forms_meet_tolerance_on_dgrad(mode, acc):
    """dX [4096, 7168] = dY [4096, 4096] . W over N = 4096, operands
    quantized by the oracle (dY per 1x128 tile along N, W per 128x128
    block and transposed), FP32 out."""
    qm = Q.POW2 if mode == "pow2" else Q.FREE
    if mode not in _DGRAD:
        w = synth.dense_up()["w"]
        dy = synth.bf16_rne(np.random.default_rng(21).standard_normal((4096, 4096)).astype(np.float32))
        say(f"[fp8-unit] dgrad operands ({mode}, oracle quantization)")
        dy_c, dy_s = Q.quantize_rows(dy, qm)
        w_c, w_s = Q.quantize_blocks(w, qm)
        _DGRAD[mode] = (dy_c, dy_s, np.ascontiguousarray(w_c.T), np.ascontiguousarray(w_s.T))
    dy_c, dy_s, wt_c, wt_s = _DGRAD[mode]
    say(f"[fp8-unit] dgrad 4096x7168 over 4096 acc={acc} scales={mode}")
    dx = host(fp8q.gemm(dev(dy_c), dev(dy_s), dev(wt_c), dev(wt_s), out_dtype=torch.float32,
                        acc=acc)).astype(np.float64)
    rng = np.random.default_rng(23)
    rows, cols = rng.integers(0, 4096, 4000), rng.integers(0, 7168, 4000)
    ref, s = G.gemm_at(dy_c, dy_s, wt_c, wt_s, rows, cols)
    ok = G.accept_f32(dx[rows, cols], ref, s)
    assert ok.all(), f"dgrad {acc} ({mode}) sampled: {int((~ok).sum())} outside the tolerance"
    for tm, tn in [(0, 1), (15, 31)]:
        r0, c0 = 256 * tm, 224 * tn
        b0, b1 = c0 // 128, (c0 + 223) // 128 + 1
        ref, s = G.gemm(dy_c[r0:r0 + 256], dy_s[r0:r0 + 256], wt_c[128 * b0:128 * b1], wt_s[b0:b1])
        ref, s = ref[:, c0 - 128 * b0:c0 - 128 * b0 + 224], s[:, c0 - 128 * b0:c0 - 128 * b0 + 224]
        got = dx[r0:r0 + 256, c0:c0 + 224]
        ok = G.accept_f32(got, ref, s)
        assert ok.all(), (f"dgrad {acc} ({mode}) tile ({tm}, {tn}): {int((~ok).sum())} of {ok.size} outside; "
                          f"max err/S {float((np.abs(got - ref) / s).max()):.3g}")


def _fraction(got, ref, s, bf16):
    ok = G.accept_bf16(got, ref, s) if bf16 else G.accept_f32(got, ref, s)
    return float(ok.mean())


def test_fp8_unit_forms_report_on_outlier_workloads():
    """Measured fractions of outputs within the stated tolerance for the
    FP8-unit forms on the workloads with outliers (a report; the float32-grade
    form is asserted by the GEMM tests)."""
    report = {}
    # tiny linear, every element
    d = synth.tiny_linear()
    for mode in ("free", "pow2"):
        qm = Q.POW2 if mode == "pow2" else Q.FREE
        a_c, a_s = Q.quantize_rows(d["a"], qm)
        w_c, w_s = Q.quantize_blocks(d["w"], qm)
        ref, s = G.gemm(a_c, a_s, w_c, w_s)
        accs = ("fp8_mfma", "fp8_mfma_scaled") if mode == "pow2" else ("fp8_mfma",)
        for acc in accs + ("fp32",):
            c = host(fp8q.gemm(dev(a_c), dev(a_s), dev(w_c), dev(w_s), out_dtype=torch.float32, acc=acc))
            report[f"tiny_128x256x512_{mode}_{acc}"] = _fraction(c.astype(np.float64), ref, s, False)
    # dense up-projection, BF16 out: 6 whole 256 x 256 tiles (rows and
    # columns spread over the output)
    d = synth.dense_up()
    rt = [0, 7, 15]
    ct = [0, 15]
    rows = np.concatenate([np.arange(256 * r, 256 * r + 256) for r in rt])
    cols = np.concatenate([np.arange(256 * c, 256 * c + 256) for c in ct])
    for mode in ("free", "pow2"):
        qm = Q.POW2 if mode == "pow2" else Q.FREE
        say(f"[fp8-unit] dense 4096x4096x7168 operands ({mode})")
        ac, as_, wc, ws = fp8q.quantize_linear(dev_bf16(d["a"]), dev_bf16(d["w"]), act_scale_mode=mode,
                                               weight_scale_mode=mode)
        oa_c, oa_s = Q.quantize_rows(d["a"][rows], qm)
        ow_c, ow_s = Q.quantize_blocks(d["w"][cols], qm)
        assert_codes_equal(host_codes(ac)[rows], oa_c, "dense A codes")
        assert_codes_equal(host_codes(wc)[cols], ow_c, "dense W codes")
        ref, s = G.gemm(oa_c, oa_s, ow_c, ow_s)
        accs = ("fp8_mfma", "fp8_mfma_scaled") if mode == "pow2" else ("fp8_mfma",)
        for acc in accs + ("fp32",):
            c = host_bf16_bits(fp8q.gemm(ac.contiguous(), as_, wc.contiguous(), ws, out_dtype=torch.bfloat16,
                                         acc=acc))
            report[f"dense_4096x4096x7168_{mode}_{acc}"] = _fraction(c[np.ix_(rows, cols)], ref, s, True)
        del ac, as_, wc, ws
    # MoE grouped (free scales), 200 sampled outputs per hosted expert
    meta, cases = moe_operands()
    offs = meta["offsets"]
    for name, (a_c, a_s, wc, ws) in cases.items():
        for acc in ("fp8_mfma", "fp32"):
            c = host_bf16_bits(fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws),
                                                 out_dtype=torch.bfloat16, acc=acc))
            rng = np.random.default_rng(9)
            oks = []
            for gi in range(len(offs) - 1):
                lo, hi = int(offs[gi]), int(offs[gi + 1])
                if hi == lo:
                    continue
                r = rng.integers(lo, hi, 200)
                q = rng.integers(0, wc.shape[1], 200)
                ref, s = G.gemm_at(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi], r - lo, q)
                oks.append(G.accept_bf16(c[r, q], ref, s))
            report[f"moe_{name}_free_{acc}"] = float(np.concatenate(oks).mean())
    say(json.dumps(report, indent=1))
    out = os.environ.get("FP8Q_UNIT_REPORT")
    if out:
        with open(out, "w") as f:
            json.dump(report, f, indent=1)
    # the float32-grade form passes everywhere it is measured here
    assert all(v == 1.0 for k, v in report.items() if k.endswith("_fp32"))
