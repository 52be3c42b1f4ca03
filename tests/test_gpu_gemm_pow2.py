"""GPU parity of the float32-grade GEMM form for power-of-two scales
(acc="fp32_pow2") against the oracle.

With power-of-two scales (tmdrlife.com wr_id=13334 ¶4) an E4M3 code times
its scale is a BF16 value, so the kernels widen each operand fragment with
its scale already applied and accumulate every K block in the BF16 matrix
core's float32 accumulator (the pages' group-scaled matrix multiply,
tmdrlife.com wr_id=13334 ¶3), with no fold.  The bar is the same as for the
default form: |gpu - oracle| <= 1e-5 * S + 1e-6 per element (BF16 output:
the interval rule), on operands the oracle quantized with power-of-two
scales.

Shapes: the tiny linear and ragged shapes (every element, both output
dtypes), all-zero tiles and tiny-amax tiles, the dense up-projection
4096 x 4096 x 7168 (sampled elements, whole rows and whole 256 x 256 tiles),
its activation gradient 4096 x 7168 over N = 4096 (224-column tiles;
sampled plus whole tiles), a MoE grouped GEMM with the workload's routing
at a reduced width (every element) and the weight gradient 2048 x 7168 over
16384 tokens (sampled plus two whole tiles).
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from oracle import gemm as G, quantize as Q
from tests.gpu_util import dev, host, host_bf16_bits, need_gpu, say
from tests.test_gpu_gemm import _accept

pytestmark = pytest.mark.gpu
P2 = Q.POW2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _gemm(a_c, a_s, w_c, w_s, out_dtype):
    return fp8q.gemm(dev(a_c), dev(a_s), dev(w_c), dev(w_s), out_dtype=out_dtype, acc="fp32_pow2")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_linear_every_element(out_dtype):
    d = synth.tiny_linear()
    a_c, a_s = Q.quantize_rows(d["a"], P2)
    w_c, w_s = Q.quantize_blocks(d["w"], P2)
    say(f"[pow2] tiny linear {out_dtype}")
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    _accept(_gemm(a_c, a_s, w_c, w_s, out_dtype), ref, s, "tiny linear")


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 5, 256), (17, 130, 384), (300, 202, 640),
                                   (511, 700, 1152), (64, 300, 128), (1000, 257, 2048)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(m, n, k, out_dtype):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    # rows spread over 2^-8 .. 2^7 so the per-row scales differ widely
    a = synth.bf16_rne((rng.standard_normal((m, k)) * np.exp2(rng.integers(-8, 8, (m, 1)))).astype(np.float32))
    w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    a_c, a_s = Q.quantize_rows(a, P2)
    w_c, w_s = Q.quantize_blocks(w, P2)
    say(f"[pow2] {m}x{n}x{k} {out_dtype}")
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    _accept(_gemm(a_c, a_s, w_c, w_s, out_dtype), ref, s, f"{m}x{n}x{k}")


def test_zero_and_tiny_tiles():
    """All-zero tiles (scale 0), tiles with max-abs near 2^-80 (scale about
    2^-89, the scaled codes still normal BF16 values) and ordinary ones in
    one operand; every element against the oracle."""
    rng = np.random.default_rng(5)
    m, n, k = 96, 160, 512
    a = rng.standard_normal((m, k)).astype(np.float32)
    a[:, 128:256] = 0.0                    # a zero tile in every row
    a[10:20] *= np.float32(2.0 ** -80)     # tiny rows
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[:, 384:] = 0.0                       # zero 128x128 blocks
    a_c, a_s = Q.quantize_rows(synth.bf16_rne(a), P2)
    w_c, w_s = Q.quantize_blocks(synth.bf16_rne(w), P2)
    assert (a_s == 0).any() and (w_s == 0).any() and (a_s[a_s > 0] < 2.0 ** -80).any()
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    _accept(_gemm(a_c, a_s, w_c, w_s, torch.float32), ref, s, "zero and tiny tiles")


def test_dense_up_projection_sampled_and_tiles():
    d = synth.dense_up()
    a_c, a_s = Q.quantize_rows(d["a"], P2)
    w_c, w_s = Q.quantize_blocks(d["w"], P2)
    say("[pow2] dense 4096x4096x7168 bf16")
    cb = host_bf16_bits(_gemm(a_c, a_s, w_c, w_s, torch.bfloat16))
    rng = np.random.default_rng(31)
    rows = np.concatenate([rng.integers(0, 4096, 4000), np.full(4096, 1234)])
    cols = np.concatenate([rng.integers(0, 4096, 4000), np.arange(4096)])
    for lo in range(0, rows.size, 4096):
        r, q = rows[lo:lo + 4096], cols[lo:lo + 4096]
        ref, s = G.gemm_at(a_c, a_s, w_c, w_s, r, q)
        ok = G.accept_bf16(cb[r, q], ref, s)
        assert ok.all(), f"pow2 dense chunk {lo}: {int((~ok).sum())} bad"
    for tm, tn in [(0, 0), (9, 4), (15, 15)]:
        r0, c0 = 256 * tm, 256 * tn
        ref, s = G.gemm(a_c[r0:r0 + 256], a_s[r0:r0 + 256], w_c[c0:c0 + 256], w_s[c0 // 128:c0 // 128 + 2])
        ok = G.accept_bf16(cb[r0:r0 + 256, c0:c0 + 256], ref, s)
        assert ok.all(), f"pow2 dense tile ({tm}, {tn}): {int((~ok).sum())} of 65536 bad"


def test_dgrad_shape_sampled_and_tiles():
    """dX [4096, 7168] = dY [4096, 4096] . W_up: the launch uses 256 x 224
    tiles, whose waves' columns cross 128-column weight-scale blocks."""
    d = synth.dense_up()
    rng = np.random.default_rng(41)
    dy = synth.bf16_rne(rng.standard_normal((4096, 4096)).astype(np.float32))
    dy_c, dy_s = Q.quantize_rows(dy, P2)
    w_c, w_s = Q.quantize_blocks(d["w"], P2)
    wt_c, wt_s = np.ascontiguousarray(w_c.T), np.ascontiguousarray(w_s.T)
    say("[pow2] dgrad 4096x7168 over 4096")
    dx = host_bf16_bits(_gemm(dy_c, dy_s, wt_c, wt_s, torch.bfloat16))
    rows, cols = rng.integers(0, 4096, 4000), rng.integers(0, 7168, 4000)
    ref, s = G.gemm_at(dy_c, dy_s, wt_c, wt_s, rows, cols)
    ok = G.accept_bf16(dx[rows, cols], ref, s)
    assert ok.all(), f"pow2 dgrad sampled: {int((~ok).sum())} bad"
    for tm, tn in [(0, 1), (15, 31)]:
        r0, c0 = 256 * tm, 224 * tn
        b0, b1 = c0 // 128, (c0 + 223) // 128 + 1
        ref, s = G.gemm(dy_c[r0:r0 + 256], dy_s[r0:r0 + 256], wt_c[128 * b0:128 * b1], wt_s[b0:b1])
        ref, s = ref[:, c0 - 128 * b0:c0 - 128 * b0 + 224], s[:, c0 - 128 * b0:c0 - 128 * b0 + 224]
        ok = G.accept_bf16(dx[r0:r0 + 256, c0:c0 + 224], ref, s)
        assert ok.all(), f"pow2 dgrad tile ({tm}, {tn}): {int((~ok).sum())} of {ok.size} bad"


def test_grouped_moe_every_element():
    """16 hosted experts with the workload's top-8 / Zipf routing over 1024
    tokens (uneven rows per expert, an empty one), hidden 512 -> 2 x 256."""
    d = synth.moe_grouped(tokens=1024, hidden=512, inter=256)
    x_c, x_s = Q.quantize_rows(d["x"], P2)
    a_c, a_s = x_c[d["gather"]], x_s[d["gather"]]
    q = [Q.quantize_blocks(d["w_up"][i], P2) for i in range(d["w_up"].shape[0])]
    wc, ws = np.stack([c for c, _ in q]), np.stack([s for _, s in q])
    offs = d["offsets"]
    say(f"[pow2] MoE up, experts {np.diff(offs).tolist()}")
    c = fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws), out_dtype=torch.bfloat16, acc="fp32_pow2")
    cb = host_bf16_bits(c)
    for gi in range(len(offs) - 1):
        lo, hi = int(offs[gi]), int(offs[gi + 1])
        if hi == lo:
            continue
        ref, s = G.gemm(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi])
        ok = G.accept_bf16(cb[lo:hi], ref, s)
        assert ok.all(), f"pow2 MoE expert {gi}: {int((~ok).sum())} of {ok.size} bad"


def test_wgrad_full_sampled_and_tiles():
    d = synth.wgrad()
    dy_c, dy_s = Q.quantize_token_t(d["dy"], P2)
    x_c, x_s = Q.quantize_token_t(d["x"], P2)
    say("[pow2] wgrad 2048x7168 over 16384 tokens")
    dw = host(fp8q.wgrad(dev(dy_c), dev(dy_s), dev(x_c), dev(x_s), acc="fp32_pow2")).astype(np.float64)
    rng = np.random.default_rng(61)
    rows, cols = rng.integers(0, 2048, 3000), rng.integers(0, 7168, 3000)
    ref, s = G.gemm_at(dy_c, dy_s, x_c, x_s, rows, cols, w_block_rows=False)
    ok = G.accept_f32(dw[rows, cols], ref, s)
    assert ok.all(), f"pow2 wgrad sampled: {int((~ok).sum())} bad"
    # two whole 256 x 224 tiles (the launch's tile width at this shape)
    for tm, tn in [(0, 0), (7, 31)]:
        r0, c0 = 256 * tm, 224 * tn
        ref, s = G.wgrad(dy_c[r0:r0 + 256], dy_s[r0:r0 + 256], x_c[c0:c0 + 224], x_s[c0:c0 + 224])
        ok = G.accept_f32(dw[r0:r0 + 256, c0:c0 + 224], ref, s)
        assert ok.all(), f"pow2 wgrad tile ({tm}, {tn}): {int((~ok).sum())} of {ok.size} bad"
