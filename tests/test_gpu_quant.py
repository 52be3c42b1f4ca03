"""GPU parity of the quantizers against the oracle: codes and scales must be
bit-identical (jp-study.kr doc 258368 ¶1; tmdrlife.com wr_id=13334 ¶4).

Covers every input of the five workloads in full: the tiny-linear and
dense-expert inputs, the quantize-only workload (16384 x 7168 activations in
both scale modes, 7168 x 18432 weights), and the weight-gradient operands
(16384 x 2048 and 16384 x 7168 in token tiles, both modes); ragged and
strided shapes, special values, the exhaustive reachable (x, amax) space of
every exponent band (against oracle digests) and of several bands element by
element, and run-to-run determinism.
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
from oracle import quantize as Q
import synth
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, dev_bf16, host, host_codes,
                            need_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _check_rows(bits, mode, what, tile_axis="row"):
    say(f"[quant] {what}: {tile_axis} {mode} shape={bits.shape}")
    codes, scales = fp8q.quantize_act(dev_bf16(bits), tile_axis=tile_axis, scale_mode=mode)
    if tile_axis == "row":
        want_c, want_s = Q.quantize_rows(bits, mode)
    else:
        want_c, want_s = Q.quantize_token_t(bits, mode)
    assert_codes_equal(host_codes(codes), want_c, what)
    assert_scales_equal(host(scales), want_s, what)


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_tiny_linear_full(mode):
    d = synth.tiny_linear()
    _check_rows(d["a"], mode, "tiny A")
    say(f"[quant] tiny W blocks {mode}")
    c, s = fp8q.quantize_weight(dev_bf16(d["w"]), scale_mode=mode)
    wc, ws = Q.quantize_blocks(d["w"], mode)
    assert_codes_equal(host_codes(c), wc, "tiny W")
    assert_scales_equal(host(s), ws, "tiny W")


def _rand_bits(rng, shape, spread=8):
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-spread, spread + 1, shape))
    return synth.bf16_rne(x.astype(np.float32))


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (2, 127), (5, 129), (17, 300), (64, 1024), (33, 640)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_ragged_rows(rows, cols, mode):
    rng = np.random.default_rng(rows * 1000 + cols)
    _check_rows(_rand_bits(rng, (rows, cols)), mode, f"ragged {rows}x{cols}")


# (700, 900) and (1500, 130): 6 x 15 and 12 x 3 workgroups, counts that the
# eight XCDs do not divide, so the block order's uneven ranges are covered;
# (300, 2040) and (1000, 4096): every XCD's range is whole groups of four
# feature groups, so the launch rotates feature groups inside each group
# (with a ragged last token block, and a ragged last feature group)
@pytest.mark.parametrize("rows,cols", [(1, 1), (128, 64), (300, 70), (129, 200), (512, 128), (256, 1000),
                                       (700, 900), (1500, 130), (300, 2040), (1000, 4096)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_ragged_token_axis(rows, cols, mode):
    rng = np.random.default_rng(rows * 7 + cols)
    _check_rows(_rand_bits(rng, (rows, cols)), mode, f"token_t {rows}x{cols}", tile_axis="token_t")


@pytest.mark.parametrize("n,k", [(1, 1), (128, 128), (200, 300), (257, 129), (384, 640)])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_ragged_blocks(n, k, mode):
    rng = np.random.default_rng(n * 13 + k)
    bits = _rand_bits(rng, (n, k))
    say(f"[quant] blocks {n}x{k} {mode}")
    c, s = fp8q.quantize_weight(dev_bf16(bits), scale_mode=mode)
    wc, ws = Q.quantize_blocks(bits, mode)
    assert_codes_equal(host_codes(c), wc, "blocks")
    assert_scales_equal(host(s), ws, "blocks")


def test_strided_input_rows_and_blocks():
    rng = np.random.default_rng(21)
    full = _rand_bits(rng, (40, 320))
    xd = dev_bf16(full)[:, :300]  # row stride 320 elements
    say("[quant] strided rows 40x300 (ld 320)")
    c, s = fp8q.quantize_act(xd, "row", "free")
    wc, ws = Q.quantize_rows(np.ascontiguousarray(full[:, :300]), "free")
    assert_codes_equal(host_codes(c), wc, "strided rows")
    assert_scales_equal(host(s), ws, "strided rows")
    c, s = fp8q.quantize_weight(xd, "pow2")
    wc, ws = Q.quantize_blocks(np.ascontiguousarray(full[:, :300]), "pow2")
    assert_codes_equal(host_codes(c), wc, "strided blocks")
    assert_scales_equal(host(s), ws, "strided blocks")


def _special_rows():
    """Tiles of zeros, negative zeros, BF16 subnormals, tiny and huge values."""
    rows = []
    z = np.zeros(256, np.uint16)
    rows.append(z.copy())
    nz = z.copy()
    nz[::3] = 0x8000  # -0
    rows.append(nz)
    sub = np.arange(256, dtype=np.uint16) % 128  # BF16 subnormals (and zeros)
    sub[1::2] |= 0x8000
    rows.append(sub)
    for ebits in (1, 2, 30, 36, 37, 38, 200, 254):  # around the normal min, the IEEE/Markstein switch, the max
        r = np.random.default_rng(ebits).integers(0, (ebits << 7) | 0x7F, 256).astype(np.uint16)
        r[0] = (ebits << 7) | 0x7F
        r[130] = (ebits << 7) | 0x60
        r[1::5] |= 0x8000
        rows.append(r)
    big = np.full(256, 0x7F7F, np.uint16)  # largest finite BF16
    big[1::2] = 0xFF7F
    rows.append(big)
    return np.stack(rows)


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_special_values(mode):
    bits = _special_rows()
    _check_rows(bits, mode, "special rows")
    _check_rows(np.ascontiguousarray(bits.T), mode, "special token_t", tile_axis="token_t")
    say(f"[quant] special blocks {mode}")
    c, s = fp8q.quantize_weight(dev_bf16(bits), scale_mode=mode)
    wc, ws = Q.quantize_blocks(bits, mode)
    assert_codes_equal(host_codes(c), wc, "special blocks")
    assert_scales_equal(host(s), ws, "special blocks")


@pytest.mark.parametrize("ebits", [0, 1, 36, 37, 100, 127, 160, 254])
@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_exhaustive_reachable_space(ebits, mode):
    bits = synth.reachable_band(ebits, seed=ebits)
    _check_rows(bits, mode, f"reachable band e={ebits}")


def _band_digests():
    from tests.conftest import golden_lines
    return {(int(e), m): (int(n), h) for e, m, n, h in golden_lines("reachable_band_digests.txt")}


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_exhaustive_reachable_space_every_band(mode):
    """All 255 BF16 exponent fields of amax, every x with |x| <= amax (530
    million (x, amax) pairs per mode): the GPU's codes and scales hash to the
    digests the oracle's quantization of the same tiles gives
    (tests/golden/make_band_digests.py).  A mismatching band is then compared
    element by element with the oracle for the report."""
    import hashlib
    want = _band_digests()
    say(f"[quant] every reachable band, {mode}")
    bad = []
    for ebits in range(255):
        bits = synth.reachable_band(ebits, seed=ebits)
        n, digest = want[(ebits, mode)]
        assert bits.shape[0] == n, (ebits, bits.shape, n)
        codes, scales = fp8q.quantize_act(dev_bf16(bits), tile_axis="row", scale_mode=mode)
        h = hashlib.sha256()
        h.update(host_codes(codes).tobytes())
        h.update(np.ascontiguousarray(host(scales), dtype="<f4").tobytes())
        if h.hexdigest() != digest:
            bad.append(ebits)
            if len(bad) == 1:  # report the first difference of the first bad band
                wc, ws = Q.quantize_rows(bits, mode)
                assert_scales_equal(host(scales), ws, f"band e={ebits} scales")
                assert_codes_equal(host_codes(codes), wc, f"band e={ebits} codes")
    assert not bad, f"bands with differences: {bad}"


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_quantize_only_activations_full(mode):
    """The quantize-only activations 16384 x 7168 (standard Student-t(3)),
    every code and scale, compared in chunks of 2048 rows."""
    act = synth.quant_only_act()
    say(f"[quant] quantize-only activations 16384x7168 {mode}, every element")
    codes, scales = fp8q.quantize_act(dev_bf16(act), "row", mode)
    sc = host(scales)
    for r0 in range(0, act.shape[0], 2048):
        wc, ws = Q.quantize_rows(act[r0:r0 + 2048], mode)
        assert_codes_equal(host_codes(codes[r0:r0 + 2048]), wc, f"act rows {r0}..")
        assert_scales_equal(sc[r0:r0 + 2048], ws, f"act rows {r0}..")


def test_quantize_only_weights_full():
    """The quantize-only weights 7168 x 18432 (~N(0, 0.02)) per 128 x 128
    block, every code and scale, compared in chunks of 8 block rows."""
    w = synth.quant_only_weight()
    say("[quant] quantize-only weights 7168x18432, every element")
    codes, scales = fp8q.quantize_weight(dev_bf16(w), "free")
    sc = host(scales)
    for bi in range(0, w.shape[0] // 128, 8):
        lo, hi = bi * 128, (bi + 8) * 128
        wc, ws = Q.quantize_blocks(w[lo:hi], "free")
        assert_codes_equal(host_codes(codes[lo:hi]), wc, f"weight block rows {bi}..{bi + 7}")
        assert_scales_equal(sc[bi:bi + 8], ws, f"weight block rows {bi}..{bi + 7}")


def test_dense_up_projection_inputs_full():
    d = synth.dense_up()
    _check_rows(d["a"], "free", "dense A 4096x7168")
    say("[quant] dense W 4096x7168 blocks")
    c, s = fp8q.quantize_weight(dev_bf16(d["w"]), "free")
    wc, ws = Q.quantize_blocks(d["w"], "free")
    assert_codes_equal(host_codes(c), wc, "dense W")
    assert_scales_equal(host(s), ws, "dense W")


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_wgrad_inputs_token_axis_full(mode):
    """The weight-gradient operands at full size, dY 16384 x 2048 and
    X 16384 x 7168 in 128-token x 1-feature tiles (codes written
    feature-major): every code and scale, in chunks of 1024 features."""
    d = synth.wgrad()
    for name in ("dy", "x"):
        bits = d[name]
        t, f = bits.shape
        say(f"[quant] wgrad {name} {t}x{f} token tiles {mode}, every element")
        codes, scales = fp8q.quantize_act(dev_bf16(bits), tile_axis="token_t", scale_mode=mode)
        sc = host(scales)
        for c0 in range(0, f, 1024):
            wc, ws = Q.quantize_token_t(np.ascontiguousarray(bits[:, c0:c0 + 1024]), mode)
            assert_codes_equal(host_codes(codes[c0:c0 + 1024]), wc, f"{name} features {c0}..")
            assert_scales_equal(sc[c0:c0 + 1024], ws, f"{name} features {c0}..")
        del codes, scales


def test_quantize_then_gather_equals_gather_then_quantize():
    """jp-study.kr doc 258368 ¶1: activations are quantized before dispatch."""
    d = synth.moe_grouped(tokens=1024, with_weights=False)
    x = dev_bf16(d["x"])
    gather = torch.from_numpy(d["gather"]).to(x.device)
    say("[quant] quantize-then-gather")
    c1, s1 = fp8q.quantize_act(x, "row", "free")
    c2, s2 = fp8q.quantize_act(x.index_select(0, gather).contiguous(), "row", "free")
    assert torch.equal(c1.index_select(0, gather), c2) and torch.equal(s1.index_select(0, gather), s2)


def test_deterministic():
    d = synth.tiny_linear()
    x = dev_bf16(d["a"])
    say("[quant] determinism")
    a = fp8q.quantize_act(x, "row", "free")
    b = fp8q.quantize_act(x, "row", "free")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


_LINEAR_CASES = [(shape, modes) for shape in ((128, 256, 512), (70, 300, 200), (0, 130, 256), (33, 0, 384))
                 for modes in (("free", "free"), ("pow2", "free"), ("free", "pow2"))] + [((4096, 4096, 7168),
                                                                                        ("free", "free"))]


@pytest.mark.parametrize("shape,modes", _LINEAR_CASES)
def test_quantize_linear_equals_separate_calls(shape, modes):
    """One launch for both operands of a linear layer: bit-identical to the
    oracle's 1x128 and 128x128 quantizations (and so to the separate calls)."""
    m, n, k = shape
    am, wm = modes
    rng = np.random.default_rng(m + 3 * n + k)
    if (m, n, k) == (4096, 4096, 7168):
        d = synth.dense_up()
        x, w = d["a"], d["w"]
    else:
        x = synth.bf16_rne((rng.standard_normal((m, k)) * np.exp2(rng.integers(-4, 5, (m, 1)))).astype(np.float32))
        w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    say(f"[quant] quantize_linear M={m} N={n} K={k} {modes}")
    ac, as_, wc, ws = fp8q.quantize_linear(dev_bf16(x), dev_bf16(w), act_scale_mode=am, weight_scale_mode=wm)
    qa = Q.POW2 if am == "pow2" else Q.FREE
    qw = Q.POW2 if wm == "pow2" else Q.FREE
    if m:
        want_c, want_s = Q.quantize_rows(x, qa)
        assert_codes_equal(host_codes(ac), want_c, "activation codes")
        assert_scales_equal(host(as_), want_s, "activation scales")
    if n:
        want_c, want_s = Q.quantize_blocks(w, qw)
        assert_codes_equal(host_codes(wc), want_c, "weight codes")
        assert_scales_equal(host(ws), want_s, "weight scales")
