"""GPU parity of the activation-gradient path (dX = dY . W) against the oracle.

jp-study.kr doc 258368 ¶3: all three GEMMs of a linear layer take FP8
inputs.  The weight is quantized once per 128x128 block; fp8q_quantize_weight_t
also writes the transposed codes and scales (W^T quantized per block equals
the transpose of W quantized, a reading the CPU tests pin), and the
activation gradient is the block-scaled GEMM of dY (1x128 tiles along N)
with that transposed operand.

Checks: the transposed codes and scales bit-exact against the oracle's block
quantization of W (both scale modes, ragged shapes, with and without the
plain copy); dX within |gpu - oracle| <= 1e-5 * S + 1e-6 (BF16: the interval
rule) every element at small sizes and sampled at the up-projection's
gradient shape (dY 4096 x 4096, W 4096 x 7168); the FP8-unit mode against
the hardware model of that unit (tests/fp8_unit_model.py, no parity claim).
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from oracle import gemm as G, quantize as Q
from tests import fp8_unit_model as unit
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, dev, dev_bf16, host, host_bf16_bits,
                            host_codes, need_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("n,k", [(1, 1), (130, 300), (256, 384), (300, 129), (128, 1000)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
@pytest.mark.parametrize("both", [True, False])
def test_transposed_weight_codes_bit_exact(n, k, mode, both):
    rng = np.random.default_rng(n * 3 + k)
    w = synth.bf16_rne((rng.standard_normal((n, k)) * np.exp2(rng.integers(-5, 6, (n, k)))).astype(np.float32))
    c_ref, s_ref = Q.quantize_blocks(w, Q.POW2 if mode == "pow2" else Q.FREE)
    say(f"[dgrad] quantize_weight_t {n}x{k} {mode} both={both}")
    c, s, ct, st = fp8q.quantize_weight_t(dev_bf16(w), scale_mode=mode, both=both)
    assert_codes_equal(host_codes(ct), c_ref.T, "codes_t")
    assert_scales_equal(host(st), s_ref.T, "scales_t")
    if both:
        assert_codes_equal(host_codes(c), c_ref, "codes")
        assert_scales_equal(host(s), s_ref, "scales")


def test_transposed_weight_codes_full_size():
    w = synth.dense_up()["w"]  # 4096 x 7168
    c_ref, s_ref = Q.quantize_blocks(w)
    say("[dgrad] quantize_weight_t 4096x7168")
    c, s, ct, st = fp8q.quantize_weight_t(dev_bf16(w))
    assert_codes_equal(host_codes(ct), c_ref.T, "codes_t")
    assert_scales_equal(host(st), s_ref.T, "scales_t")
    assert_codes_equal(host_codes(c), c_ref, "codes")
    # the plain copy is the one fp8q_quantize_weight writes
    c2, s2 = fp8q.quantize_weight(dev_bf16(w))
    assert torch.equal(c, c2) and torch.equal(s, s2)


def _operands(dy_bits, w_bits):
    dy_c, dy_s = Q.quantize_rows(dy_bits)        # 1x128 tiles along N
    w_c, w_s = Q.quantize_blocks(w_bits)        # [N, K] blocks
    return dy_c, dy_s, np.ascontiguousarray(w_c.T), np.ascontiguousarray(w_s.T)


@pytest.mark.parametrize("m,n,k", [(1, 128, 1), (70, 256, 130), (300, 384, 520)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dgrad_small_every_element(m, n, k, out_dtype):
    rng = np.random.default_rng(m + 5 * n + k)
    dy = synth.bf16_rne(rng.standard_normal((m, n)).astype(np.float32))
    w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    dy_c, dy_s, wt_c, wt_s = _operands(dy, w)
    say(f"[dgrad] dX {m}x{k}, N={n} {out_dtype}")
    # the device operand comes from the library's own transposed quantizer
    _, _, ct, st = fp8q.quantize_weight_t(dev_bf16(w), both=False)
    assert_codes_equal(host_codes(ct), wt_c, "codes_t")
    dx = fp8q.dgrad(dev(dy_c), dev(dy_s), ct.contiguous(), st, out_dtype=out_dtype)
    ref, s = G.gemm(dy_c, dy_s, wt_c, wt_s)
    if out_dtype == torch.bfloat16:
        ok = G.accept_bf16(host_bf16_bits(dx), ref, s)
    else:
        ok = G.accept_f32(host(dx).astype(np.float64), ref, s)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outside tolerance"


def test_dgrad_up_projection_sampled():
    """dX [4096 tokens, 7168] = dY [4096, 4096] . W_up [4096, 7168]."""
    d = synth.dense_up()
    rng = np.random.default_rng(21)
    dy = synth.bf16_rne(rng.standard_normal((4096, 4096)).astype(np.float32))
    dy_c, dy_s, wt_c, wt_s = _operands(dy, d["w"])
    say("[dgrad] dX 4096x7168 over N=4096, bf16 out, both accumulation modes")
    for acc in ("fp32", "fp8_mfma"):
        dx = host_bf16_bits(fp8q.dgrad(dev(dy_c), dev(dy_s), dev(wt_c), dev(wt_s), out_dtype=torch.bfloat16,
                                       acc=acc))
        rows = np.concatenate([rng.integers(0, 4096, 4000), np.full(7168, 4095)])
        cols = np.concatenate([rng.integers(0, 7168, 4000), np.arange(7168)])
        for lo in range(0, rows.size, 4096):
            r, q = rows[lo:lo + 4096], cols[lo:lo + 4096]
            if acc == "fp32":
                ref, s = G.gemm_at(dy_c, dy_s, wt_c, wt_s, r, q)
            else:
                ref, s, t = unit.gemm_at_mfma(dy_c, dy_s, wt_c, wt_s, r, q)
                s = s + (2.0 ** -19) * t / 1e-5
            ok = G.accept_bf16(dx[r, q], ref, s)
            assert ok.all(), f"dgrad {acc} chunk {lo}: {int((~ok).sum())} bad"
        if acc == "fp32":
            # every element of whole output tiles: at this shape the launch
            # uses tiles of 256 x 224 (512 of them fill the 256 CUs in two
            # rounds), whose waves' 112 columns start inside a 128-column
            # weight-scale block (tile 1: columns 224..447) or end the
            # matrix (tile 31: columns 6944..7167)
            for tm, tn in [(0, 1), (7, 10), (15, 31)]:
                r0, c0 = 256 * tm, 224 * tn
                # the oracle over the 128-aligned columns around the tile
                # (weight-scale row b covers columns 128b..128b+127)
                b0, b1 = c0 // 128, (c0 + 223) // 128 + 1
                ref, s = G.gemm(dy_c[r0:r0 + 256], dy_s[r0:r0 + 256], wt_c[128 * b0:128 * b1], wt_s[b0:b1])
                ref, s = ref[:, c0 - 128 * b0:c0 - 128 * b0 + 224], s[:, c0 - 128 * b0:c0 - 128 * b0 + 224]
                ok = G.accept_bf16(dx[r0:r0 + 256, c0:c0 + 224], ref, s)
                assert ok.all(), f"dgrad tile ({tm}, {tn}): {int((~ok).sum())} of {ok.size} bad"
