"""GPU parity at the largest sizes the entry points accept, where element
and byte offsets pass 2^31 and 2^32.

The quantizers and the SwiGLU pass take each size below 2^31 and are
limited only by memory; here their inputs reach 4.7-9.2 GB and their codes
2.2-4.6 GB.  The GEMMs and the gather take operands below 2 GiB each; here
each operand in turn sits just below that limit (A, W, the grouped weights
of all experts, the Wgrad X^T, the gather source).

Inputs.  A seeded host block from ``synth`` is tiled over the rows on the
GPU (torch ``repeat``); for the BF16 inputs each row (token, for the token
axis) is then multiplied by 1 + (r mod 7) / 8, so rows differ and the input
repeats with period lcm(block rows, 7).  GEMM and gather operands are
uniformly drawn finite E4M3 codes tiled the same way, with a free float32
scale per tile drawn for every row (no period).

Checks.
* Sampled rows (features, block rows, output columns) against the oracle,
  on the device values copied back: the first rows, rows on either side of
  the element offset 2^31 and of the code byte offset 2^32 where the shape
  reaches them, the last rows.  Codes and scales bit-exact; GEMM outputs
  within |gpu - oracle| <= 1e-5 * S + 1e-6; SwiGLU tiles by the oracle's
  acceptance rule (bit-exact up to BF16 rounding-midpoint ambiguity).
* At full size, on the device, for the quantizers and SwiGLU: the outputs
  were pre-filled with a NaN code (0xFF) and NaN scales, which no call
  writes, so none may remain; and outputs repeat with the input's period, so
  a row written to the wrong place or not at all breaks the repetition.
"""

import ctypes

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from oracle import gemm as G, moe, quantize as Q
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, dev, dev_bf16, host, host_bf16_bits,
                            host_codes, need_gpu, say)

pytestmark = pytest.mark.gpu
MODE = {"free": fp8q.SCALE_FREE, "pow2": fp8q.SCALE_POW2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.empty_cache()


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _vp(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _tiled_bf16(block_bits, reps, rows, axis_period=7):
    """block tiled over the rows on the GPU, row r scaled by 1 + (r % 7) / 8."""
    x = dev_bf16(block_bits).repeat(reps, 1)[:rows]
    f = (1.0 + (torch.arange(rows, device="cuda:0") % axis_period).to(torch.float32) / 8.0).to(torch.bfloat16)
    x.mul_(f.unsqueeze(1))
    return x


def _sentinel_codes(shape):
    return torch.full(shape, 0xFF, dtype=torch.uint8, device="cuda:0")


def _sentinel_scales(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda:0")


def _no_sentinel(codes, scales, what):
    assert not bool(((codes & 0x7F) == 0x7F).any()), f"{what}: a NaN code is left (an element not written)"
    assert bool(torch.isfinite(scales).all()), f"{what}: a NaN scale is left (a tile not written)"


def _periodic(t, period, dim, what):
    n = t.shape[dim]
    a, b = t.narrow(dim, period, n - period), t.narrow(dim, 0, n - period)
    assert torch.equal(a, b), f"{what}: output does not repeat with the input's period {period}"


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_row_quantizer_codes_past_4_gib(mode):
    """1x128 tiles of x [640000, 7168]: 9.2 GB in, 4.6 GB of codes."""
    rows, cols = 640000, 7168
    rng = np.random.default_rng(71)
    block = synth.bf16_rne(rng.standard_t(3, (1000, cols)).astype(np.float32))
    say(f"[max] row quantizer {rows}x{cols} {mode}")
    x = _tiled_bf16(block, 640, rows)
    codes, scales = _sentinel_codes((rows, cols)), _sentinel_scales((rows, cols // 128))
    st = fp8q.load_library().fp8q_quantize_act(_vp(x), rows, cols, cols, fp8q.TILE_ROW, MODE[mode], _vp(codes), cols,
                                               _vp(scales), _stream())
    assert st == fp8q.OK, fp8q.status_string(st)
    _no_sentinel(codes, scales, "row codes")
    _periodic(codes, 7000, 0, "row codes")
    _periodic(scales, 7000, 0, "row scales")
    # 2^31 elements: row 299593; 2^32 code bytes: row 599186
    pick = [0, 1, 999, 1000, 6999, 7000, 299592, 299593, 299594, 599185, 599186, 599187, rows - 2, rows - 1]
    want_c, want_s = Q.quantize_rows(host_bf16_bits(x[pick]), Q.POW2 if mode == "pow2" else Q.FREE)
    assert_codes_equal(host_codes(codes[pick]), want_c, "row codes (sampled rows)")
    assert_scales_equal(host(scales[pick]), want_s, "row scales (sampled rows)")


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_token_axis_quantizer_past_4_gib(mode):
    """128x1 token tiles of x [327680 tokens, 7168]: 4.7 GB in, transposed
    codes [7168, 327680] of 2.35 GB."""
    t, c = 327680, 7168
    rng = np.random.default_rng(72)
    block = synth.bf16_rne(rng.standard_normal((4096, c)).astype(np.float32))
    say(f"[max] token-axis quantizer {t}x{c} {mode}")
    x = _tiled_bf16(block, 80, t)
    codes, scales = _sentinel_codes((c, t)), _sentinel_scales((c, t // 128))
    st = fp8q.load_library().fp8q_quantize_act(_vp(x), t, c, c, fp8q.TILE_TOKEN_T, MODE[mode], _vp(codes), t,
                                               _vp(scales), _stream())
    assert st == fp8q.OK, fp8q.status_string(st)
    _no_sentinel(codes, scales, "token codes")
    _periodic(codes, 28672, 1, "token codes")      # lcm(4096, 7) tokens
    _periodic(scales, 224, 1, "token scales")
    # features 6553 / 6554 hold code byte offset 2^31; every column reaches
    # input element offsets past 2^31 in its last tokens
    feats = [0, 1, 63, 64, 3583, 6553, 6554, c - 1]
    want_c, want_s = Q.quantize_token_t(host_bf16_bits(x[:, feats]), Q.POW2 if mode == "pow2" else Q.FREE)
    assert_codes_equal(host_codes(codes[feats]), want_c, "token codes (sampled features)")
    assert_scales_equal(host(scales[feats]), want_s, "token scales (sampled features)")


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_block_quantizer_past_2_gib(mode):
    """128x128 blocks of w [300032, 7168]: 4.3 GB in, 2.15 GB of codes."""
    n, k = 300032, 7168
    rng = np.random.default_rng(73)
    block = synth.bf16_rne(rng.standard_normal((1024, k)).astype(np.float32) * np.float32(0.02))
    say(f"[max] block quantizer {n}x{k} {mode}")
    w = _tiled_bf16(block, 293, n)
    codes, scales = _sentinel_codes((n, k)), _sentinel_scales((n // 128, k // 128))
    st = fp8q.load_library().fp8q_quantize_weight(_vp(w), n, k, k, MODE[mode], _vp(codes), k, _vp(scales), _stream())
    assert st == fp8q.OK, fp8q.status_string(st)
    _no_sentinel(codes, scales, "block codes")
    _periodic(codes, 7168, 0, "block codes")       # lcm(1024, 7) rows
    _periodic(scales, 56, 0, "block scales")
    for br in (0, 1, 1170, 2340, n // 128 - 1):    # block row 2340 crosses element 2^31
        r0 = 128 * br
        want_c, want_s = Q.quantize_blocks(host_bf16_bits(w[r0:r0 + 128]), Q.POW2 if mode == "pow2" else Q.FREE)
        assert_codes_equal(host_codes(codes[r0:r0 + 128]), want_c, f"block codes (block row {br})")
        assert_scales_equal(host(scales[br:br + 1]), want_s, f"block scales (block row {br})")


def _accept(got, ref, s, what):
    ok = G.accept_f32(got, ref, s)
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outside the tolerance"


def test_gemm_activation_operand_at_limit():
    """A [299593, 7168] (2^31 - 1024 bytes) . W [384, 7168]^T -> FP32."""
    m, n, k = 299593, 384, 7168
    rng = np.random.default_rng(74)
    a_blk = synth.e4m3_codes(rng, (1000, k))
    a_s = synth.tile_scales(rng, (m, k // 128))
    w_c = synth.e4m3_codes(rng, (n, k))
    w_s = synth.tile_scales(rng, (3, k // 128))
    say(f"[max] gemm A {m}x{k} (bytes {m * k})")
    a = dev(a_blk).repeat(300, 1)[:m]
    c = host(fp8q.gemm(a, dev(a_s), dev(w_c), dev(w_s), out_dtype=torch.float32)).astype(np.float64)
    # the last, ragged row tile (73 rows) and the row tile past 2^30 bytes, every column
    for r0, r1 in ((299520, m), (149760, 149760 + 256)):
        rows = np.arange(r0, r1)
        ref, s = G.gemm(a_blk[rows % 1000], a_s[rows], w_c, w_s)
        _accept(c[r0:r1], ref, s, f"gemm rows {r0}..{r1 - 1}")


def test_gemm_weight_operand_at_limit():
    """A [300, 7168] . W [299593, 7168]^T (W 2^31 - 1024 bytes) -> FP32."""
    m, n, k = 300, 299593, 7168
    rng = np.random.default_rng(75)
    a_c = synth.e4m3_codes(rng, (m, k))
    a_s = synth.tile_scales(rng, (m, k // 128))
    w_blk = synth.e4m3_codes(rng, (1024, k))
    w_s = synth.tile_scales(rng, ((n + 127) // 128, k // 128))
    say(f"[max] gemm W {n}x{k} (bytes {n * k})")
    w = dev(w_blk).repeat(293, 1)[:n]
    c = host(fp8q.gemm(dev(a_c), dev(a_s), w, dev(w_s), out_dtype=torch.float32)).astype(np.float64)
    for blk in (0, 1170, (n - 1) // 128):          # the last block holds 73 columns
        cols = np.arange(128 * blk, min(n, 128 * blk + 128))
        ref, s = G.gemm(a_c, a_s, w_blk[cols % 1024], w_s[blk:blk + 1])
        _accept(c[:, cols], ref, s, f"gemm column block {blk}")


def test_grouped_gemm_weights_at_limit():
    """Two experts of W [149796, 7168] each (all weights 2^31 - 8192 bytes),
    100 and 37 rows."""
    g, n, k = 2, 149796, 7168
    rng = np.random.default_rng(76)
    a_c = synth.e4m3_codes(rng, (200, k))
    a_s = synth.tile_scales(rng, (200, k // 128))
    w_blk = synth.e4m3_codes(rng, (1024, k))
    w_s = synth.tile_scales(rng, (g, (n + 127) // 128, k // 128))
    offs = np.array([0, 100, 137], dtype=np.int32)
    say(f"[max] grouped gemm {g} x {n}x{k} (bytes {g * n * k})")
    w = dev(w_blk).repeat(293, 1)[:g * n].view(g, n, k)
    c = host(fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), w, dev(w_s), out_dtype=torch.float32))
    c = c.astype(np.float64)
    for gi in range(g):
        lo, hi = int(offs[gi]), int(offs[gi + 1])
        for blk in (0, (n - 1) // 128):            # the last block holds 36 columns
            cols = np.arange(128 * blk, min(n, 128 * blk + 128))
            ref, s = G.gemm(a_c[lo:hi], a_s[lo:hi], w_blk[(gi * n + cols) % 1024], w_s[gi, blk:blk + 1])
            _accept(c[lo:hi][:, cols], ref, s, f"expert {gi} column block {blk}")


def test_wgrad_x_operand_at_limit():
    """dW [300, 16383] over T = 131072 tokens; X^T [16383, 131072] is
    2^31 - 131072 bytes."""
    nout, kin, t = 300, 16383, 131072
    rng = np.random.default_rng(77)
    dy_c = synth.e4m3_codes(rng, (nout, t))
    dy_s = synth.tile_scales(rng, (nout, t // 128))
    x_blk = synth.e4m3_codes(rng, (1000, t))
    x_s = synth.tile_scales(rng, (kin, t // 128))
    say(f"[max] wgrad X^T {kin}x{t} (bytes {kin * t})")
    x = dev(x_blk).repeat(17, 1)[:kin]
    dw = host(fp8q.wgrad(dev(dy_c), dev(dy_s), x, dev(x_s))).astype(np.float64)
    for c0, c1 in ((0, 32), (16352, kin)):         # the last 224-column tile holds 31 columns
        cols = np.arange(c0, c1)
        ref, s = G.wgrad(dy_c, dy_s, x_blk[cols % 1000], x_s[cols])
        _accept(dw[:, cols], ref, s, f"wgrad columns {c0}..{c1 - 1}")


def test_gather_source_at_limit():
    """Gather 4099 rows from codes [299593, 7168] (2^31 - 1024 bytes)."""
    rows, cols = 299593, 7168
    rng = np.random.default_rng(78)
    blk = synth.e4m3_codes(rng, (1000, cols))
    sc = synth.tile_scales(rng, (rows, cols // 128))
    idx = np.concatenate([rng.integers(0, rows, 4096), [0, rows - 1, rows - 2]]).astype(np.int32)
    say(f"[max] gather from {rows}x{cols}")
    src = dev(blk).repeat(300, 1)[:rows]
    gc, gs = fp8q.gather_rows(src, dev(sc), dev(idx))
    want_c, _ = moe.gather_rows(blk, np.zeros((1000, cols // 128), np.float32), idx % 1000)
    _, want_s = moe.gather_rows(np.zeros((rows, 0), np.uint8), sc, idx)
    assert_codes_equal(host_codes(gc), want_c, "gathered codes")
    assert_scales_equal(host(gs), want_s, "gathered scales")


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_swiglu_input_past_4_gib(mode):
    """SwiGLU + 1x128 quantize of x [300000, 2 x 4096]: 4.9 GB in."""
    rows, inter = 300000, 4096
    rng = np.random.default_rng(79)
    block = synth.bf16_rne(rng.standard_normal((1000, 2 * inter)).astype(np.float32) * np.float32(1.7))
    say(f"[max] swiglu {rows}x{inter} {mode}")
    x = _tiled_bf16(block, 300, rows)
    codes, scales = _sentinel_codes((rows, inter)), _sentinel_scales((rows, inter // 128))
    st = fp8q.load_library().fp8q_swiglu_quantize(_vp(x), rows, inter, 2 * inter, MODE[mode], _vp(codes), inter,
                                                  _vp(scales), 0, None, 0, None, _stream())
    assert st == fp8q.OK, fp8q.status_string(st)
    _no_sentinel(codes, scales, "swiglu codes")
    _periodic(codes, 7000, 0, "swiglu codes")
    _periodic(scales, 7000, 0, "swiglu scales")
    # input element offset 2^31: row 262144
    pick = [0, 999, 1000, 6999, 7000, 262143, 262144, rows - 1]
    ok = moe.swiglu_accept(host_bf16_bits(x[pick]), mode, host_codes(codes[pick]), host(scales[pick]))
    assert ok.all(), f"swiglu: {int((~ok).sum())} of {ok.size} sampled tiles rejected"
