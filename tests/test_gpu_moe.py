"""GPU parity of the MoE glue against the oracle.

FP8 dispatch gather (jp-study.kr doc 258368 ¶1): codes and scales bit-exact
against oracle.moe.gather_rows -- the hosted rows of the 8192-token MoE
workload in full, ragged column counts (16-byte and element-wise paths),
strided sources, repeated and out-of-range indices, an empty source and an
empty index list.

SwiGLU + 1x128 quantization (tmdrlife.com wr_id=13334 ¶3-¶4): every tile must
pass oracle.moe.swiglu_accept (codes and scale bit-exact, except that an
element whose exact SwiGLU value lies within 2^-19 of a BF16 rounding
midpoint may take either neighbour); tiles with no such element are also
compared directly with the oracle's quantization.  The optional cache of the
input is bit-exact against the oracle's 1x128 quantization of the input and
against fp8q.quantize_act.  Shapes: ragged inter (1, 100, 130), multiples of
128, a strided input, special gate values, gate ranges that put the kernel
in each of its two float32 forms, and the MoE workload's [3773, 2 x 2048]
up-projection output shape in full.
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
from oracle import moe, quantize as Q
from oracle.e4m3 import bf16_bits_to_f32
import synth
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, dev, dev_bf16, host, host_codes,
                            need_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _random_codes(rng, rows, cols):
    """Codes and scales of a quantized random activation (oracle-side)."""
    x = synth.bf16_rne((rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 7, (rows, 1)))).astype(np.float32))
    return Q.quantize_rows(x)


@pytest.mark.parametrize("rows,cols,n_out", [(10, 128, 7), (37, 100, 50), (5, 1, 9), (64, 7168, 130),
                                             (3, 17, 4), (20, 256, 0)])
def test_gather_small(rows, cols, n_out):
    rng = np.random.default_rng(rows * 31 + cols)
    c, s = _random_codes(rng, rows, cols)
    idx = rng.integers(-2, rows + 2, n_out).astype(np.int32)  # includes out-of-range rows
    say(f"[moe] gather rows={rows} cols={cols} n_out={n_out}")
    gc, gs = fp8q.gather_rows(dev(c), dev(s), dev(idx))
    wc, ws = moe.gather_rows(c, s, idx)
    assert_codes_equal(host_codes(gc), wc, "gathered codes")
    assert_scales_equal(host(gs), ws, "gathered scales")


def test_gather_strided_source_and_empty_source():
    rng = np.random.default_rng(5)
    c, s = _random_codes(rng, 30, 200)
    buf = np.zeros((30, 224), dtype=np.uint8)
    buf[:, :200] = c
    src = dev(buf)[:, :200]  # row stride 224 bytes
    idx = np.array([29, 0, 0, 15, 31, -5], dtype=np.int32)
    say("[moe] gather strided source")
    gc, gs = fp8q.gather_rows(src, dev(s), dev(idx))
    wc, ws = moe.gather_rows(c, s, idx)
    assert_codes_equal(host_codes(gc), wc, "strided gather")
    assert_scales_equal(host(gs), ws, "strided gather scales")
    say("[moe] gather from an empty source")
    empty_c = torch.empty((0, 200), dtype=torch.uint8, device="cuda:0")
    empty_s = torch.empty((0, 2), dtype=torch.float32, device="cuda:0")
    gc, gs = fp8q.gather_rows(empty_c, empty_s, dev(np.array([0, 3], dtype=np.int32)))
    assert not host_codes(gc).any() and not host(gs).any()


def test_gather_moe_dispatch_full():
    """The hosted rows of the 8192-token workload, quantized once and
    gathered by expert."""
    d = synth.moe_grouped(with_weights=False)
    idx = d["gather"].astype(np.int32)
    say(f"[moe] dispatch gather: 8192 x 7168 -> {idx.size} rows")
    xq, xs = fp8q.quantize_act(dev_bf16(d["x"]))
    gc, gs = fp8q.gather_rows(xq, xs, dev(idx))
    # the source codes are the oracle's (bit-exact quantizer), so the
    # expected rows are the oracle's quantization of the gathered tokens
    wc, ws = Q.quantize_rows(d["x"][idx])
    assert_codes_equal(host_codes(gc), wc, "dispatch codes")
    assert_scales_equal(host(gs), ws, "dispatch scales")


def _check_swiglu(x_bits, mode, what, x_dev=None, cache=False, cache_mode="pow2"):
    xd = dev_bf16(x_bits) if x_dev is None else x_dev
    out = fp8q.swiglu_quantize(xd, scale_mode=mode, cache=cache, cache_scale_mode=cache_mode)
    c, s = host_codes(out[0]), host(out[1])
    ok = moe.swiglu_accept(x_bits, mode, c, s)
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{what}: {len(bad)} of {ok.size} tiles rejected, first {tuple(bad[0])}"
    c1, c2 = moe.swiglu_candidates(x_bits)
    amb = c1 != c2
    wc, ws = moe.swiglu_quantize(x_bits, mode)
    inter = c1.shape[1]
    nb = s.shape[1]
    # tiles without an ambiguous element: bit-exact
    clean = np.ones(ok.shape, dtype=bool)
    for b in range(nb):
        clean[:, b] = ~amb[:, b * 128:min(inter, (b + 1) * 128)].any(axis=1)
    rows_clean = np.repeat(clean, 128, axis=1)[:, :inter]
    assert np.array_equal(np.where(rows_clean, c, 0), np.where(rows_clean, wc, 0)), what
    assert np.array_equal(np.where(clean, s, 0).view(np.uint32), np.where(clean, ws, 0).view(np.uint32)), what
    say(f"[moe] {what}: {ok.size} tiles accepted, {int(amb.sum())} elements near a BF16 midpoint")
    if cache:
        cc, cs = host_codes(out[2]), host(out[3])
        want_c, want_s = Q.quantize_rows(x_bits, cache_mode)
        assert_codes_equal(cc, want_c, what + " cache codes")
        assert_scales_equal(cs, want_s, what + " cache scales")
        qc, qs = fp8q.quantize_act(xd, scale_mode=cache_mode)
        assert torch.equal(out[2], qc) and torch.equal(out[3], qs)


@pytest.mark.parametrize("rows,inter", [(1, 1), (7, 100), (33, 130), (64, 128), (300, 512), (5, 2048)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_swiglu_small(rows, inter, mode):
    rng = np.random.default_rng(rows * 7 + inter)
    x = synth.bf16_rne((rng.standard_normal((rows, 2 * inter)) * np.exp2(rng.integers(-3, 4, (rows, 1)))).astype(np.float32))
    say(f"[moe] swiglu {rows}x{inter} {mode}")
    _check_swiglu(x, mode, f"swiglu {rows}x{inter} {mode}", cache=(inter % 128 == 0),
                  cache_mode="pow2" if mode == "free" else "free")


def test_swiglu_strided_and_special_values():
    rng = np.random.default_rng(9)
    inter = 256
    g = rng.standard_normal((16, inter)).astype(np.float32)
    special = np.array([0.0, -0.0, 1.0, -1.0, 40.0, -40.0, 80.0, -80.0, -100.0, 3.0, -3.0, 0.5], dtype=np.float32)
    g[:, :special.size] = special
    u = rng.standard_normal((16, inter)).astype(np.float32)
    u[0, :] = 0.0
    u[1, :] = -0.0
    u[2, :special.size] = 1.0
    x = synth.bf16_rne(np.concatenate([g, u], axis=1))
    buf = np.zeros((16, 2 * inter + 64), dtype=np.uint16)
    buf[:, :2 * inter] = x
    xd = dev_bf16(buf)[:, :2 * inter]  # row stride 576 elements
    for mode in ("free", "pow2"):
        say(f"[moe] swiglu special values, strided input, {mode}")
        _check_swiglu(x, mode, f"swiglu special {mode}", x_dev=xd, cache=True)


def test_swiglu_gate_ranges_of_both_forms():
    """The kernel forms a chunk's values in one of two float32 ways, chosen
    per wave: the direct one when every gate of the wave's chunks is at
    least -64, the general one otherwise.  Rows 0-31 hold gates in
    [-64, -40] (the direct form's largest e^-g, -64 itself included),
    rows 32-63 gates in [40, 1000]; rows 64-127 are the same draws with a
    single gate in [-104, -64) planted in every fourth tile, so those waves
    take the general form for all four of their tiles."""
    rng = np.random.default_rng(21)
    inter = 512
    g = np.concatenate([rng.uniform(-64, -40, (32, inter)), rng.uniform(40, 1000, (32, inter))])
    g[0, :4] = [-64.0, -63.75, -40.0, -50.5]
    g = np.concatenate([g, g]).astype(np.float32)
    for r in range(64, 128):
        g[r, 128 * (r % 4) + (r * 7) % 128] = -rng.uniform(64.5, 104)
    u = (rng.standard_normal((128, inter)) * np.exp2(rng.integers(-2, 3, (128, 1)))).astype(np.float32)
    x = synth.bf16_rne(np.concatenate([g, u], axis=1))
    gv = bf16_bits_to_f32(x[:, :inter])
    assert gv[:64].min() >= -64 and (gv[64:] < -64).sum() == 64
    for mode in ("free", "pow2"):
        say(f"[moe] swiglu gate ranges of both forms, {mode}")
        _check_swiglu(x, mode, f"swiglu gate ranges {mode}", cache=True)


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_swiglu_moe_workload_full(mode):
    x = synth.swiglu_input()
    say(f"[moe] swiglu {x.shape[0]}x{x.shape[1] // 2} (MoE up-projection output) {mode}")
    _check_swiglu(x, mode, f"swiglu MoE {mode}", cache=True)
