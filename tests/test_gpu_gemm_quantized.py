"""GPU parity of the GEMM with an FP8 epilogue (fp8q_gemm_quantized).

tmdrlife.com wr_id=13334 ¶1: the BF16 output of one computation is read back
only to be quantized for the next FP8 MMA; the producer here writes the
1x128-quantized form directly.

Checks:
* parity with the oracle: every 1x128 tile of the output passes
  oracle.gemm.accept_quantized -- it is the 1x128 quantization of a BF16
  tensor within |c - C| <= 1e-5 * S + 1e-6 of the exact product -- for every
  tile at small and ragged shapes and for whole sampled rows of the dense
  up-projection 4096 x 4096 x 7168, in both scale modes;
* the fusion changes nothing: the codes and scales are bit-identical to
  fp8q.gemm(BF16 out) on 256-wide tiles (the tiling the fused kernel has)
  followed by fp8q.quantize_act, in every accumulation form, at the full
  dense size and at 333 x 520 x 256, a size the float32-grade fp8q.gemm
  would otherwise run on 32 x 32 split-K tiles.
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
from oracle import gemm as G, quantize as Q
import synth
from tests.gpu_util import assert_codes_equal, assert_scales_equal, dev, dev_bf16, host, host_codes, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _operands(rng, m, n, k, mode=Q.FREE, outliers=False):
    a = rng.standard_normal((m, k)).astype(np.float32)
    if outliers:
        a[rng.random((m, k)) < 0.001] *= 100
    a = synth.bf16_rne(a)
    w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    ac, as_ = Q.quantize_rows(a, mode)
    wc, ws = Q.quantize_blocks(w, mode)
    return ac, as_, wc, ws


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (70, 256, 384), (300, 384, 512), (256, 200, 256),
                                   (130, 1, 128), (64, 520, 1024), (5, 300, 0)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_small_every_tile(m, n, k, mode):
    rng = np.random.default_rng(m * 13 + n * 7 + k)
    qm = Q.POW2 if mode == "pow2" else Q.FREE
    ac, as_, wc, ws = _operands(rng, m, n, k, outliers=True)
    say(f"[gemm-q] {m}x{n}x{k} {mode}")
    codes, scales = fp8q.gemm_quantized(dev(ac), dev(as_), dev(wc), dev(ws), scale_mode=mode)
    c, s = G.gemm(ac, as_, wc, ws)
    ok = G.accept_quantized(host_codes(codes), host(scales), c, s, qm)
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{len(bad)} of {ok.size} tiles rejected, first {tuple(bad[0])}"


@pytest.mark.parametrize("m,n,k", [(70, 256, 384), (300, 384, 512), (64, 520, 1024)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_small_every_tile_fp32_pow2(m, n, k, mode):
    """The float32-grade form for power-of-two operand scales writing the
    quantized output (output tiles in either scale mode)."""
    rng = np.random.default_rng(m * 17 + n * 5 + k)
    qm = Q.POW2 if mode == "pow2" else Q.FREE
    a = synth.bf16_rne(rng.standard_normal((m, k)).astype(np.float32))
    w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    ac, as_ = Q.quantize_rows(a, Q.POW2)
    wc, ws = Q.quantize_blocks(w, Q.POW2)
    say(f"[gemm-q] {m}x{n}x{k} out {mode}, acc fp32_pow2")
    codes, scales = fp8q.gemm_quantized(dev(ac), dev(as_), dev(wc), dev(ws), scale_mode=mode, acc="fp32_pow2")
    c, s = G.gemm(ac, as_, wc, ws)
    ok = G.accept_quantized(host_codes(codes), host(scales), c, s, qm)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} tiles rejected"


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_dense_up_projection_sampled_rows(mode):
    d = synth.dense_up()
    qm = Q.POW2 if mode == "pow2" else Q.FREE
    ac, as_ = Q.quantize_rows(d["a"])
    wc, ws = Q.quantize_blocks(d["w"])
    say(f"[gemm-q] 4096x4096x7168 {mode}, whole sampled rows")
    codes, scales = fp8q.gemm_quantized(dev(ac), dev(as_), dev(wc), dev(ws), scale_mode=mode)
    codes, scales = host_codes(codes), host(scales)
    rows = np.array([0, 1, 777, 2048, 4095])
    cols = np.arange(4096)
    r = np.repeat(rows, cols.size)
    q = np.tile(cols, rows.size)
    ref, s = G.gemm_at(ac, as_, wc, ws, r, q)
    ok = G.accept_quantized(codes[rows], scales[rows], ref.reshape(rows.size, -1), s.reshape(rows.size, -1), qm)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} tiles rejected"


@pytest.mark.parametrize("acc", ["fp32", "fp8_mfma", "fp8_mfma_scaled", "fp32_pow2"])
def test_fused_equals_gemm_then_quantize(acc):
    rng = np.random.default_rng(3)
    for m, n, k in ((4096, 4096, 7168), (333, 520, 256)):
        mode = Q.POW2 if acc in ("fp8_mfma_scaled", "fp32_pow2") else Q.FREE
        if (m, n, k) == (4096, 4096, 7168) and mode == Q.FREE:
            d = synth.dense_up()
            a, w = dev_bf16(d["a"]), dev_bf16(d["w"])
        else:
            a = dev_bf16(synth.bf16_rne(rng.standard_normal((m, k)).astype(np.float32)))
            w = dev_bf16(synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32)))
        ac, as_ = fp8q.quantize_act(a, scale_mode=mode)
        wc, ws = fp8q.quantize_weight(w, scale_mode=mode)
        ac, wc = ac.contiguous(), wc.contiguous()
        for out_mode in ("free", "pow2"):
            say(f"[gemm-q] fused vs unfused {m}x{n}x{k} acc={acc} out={out_mode}")
            codes, scales = fp8q.gemm_quantized(ac, as_, wc, ws, scale_mode=out_mode, acc=acc)
            prev = fp8q.set_gemm_small_limit(0)
            try:
                c = fp8q.gemm(ac, as_, wc, ws, out_dtype=torch.bfloat16, acc=acc)
            finally:
                fp8q.set_gemm_small_limit(prev)
            want_c, want_s = fp8q.quantize_act(c, scale_mode=out_mode)
            assert_codes_equal(host_codes(codes), host_codes(want_c), "fused codes")
            assert_scales_equal(host(scales), host(want_s), "fused scales")
