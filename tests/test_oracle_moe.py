"""Pins for the oracle's MoE glue (CPU): the FP8 dispatch gather and the
SwiGLU + 1x128 quantization (jp-study.kr doc 258368 ¶1; tmdrlife.com
wr_id=13334 ¶3-¶4).

What is checked without re-deriving the oracle's own formulas:

* a hand-worked gather, with repeated and out-of-range indices;
* gathering the codes of quantized rows equals quantizing the gathered BF16
  rows (the 1x128 tiles are per row, so dispatching FP8 loses nothing);
* silu closed forms: silu(0) = 0, sigmoid(ln 3) = 3/4, silu(x) - silu(-x) = x,
  silu(x) -> x for large x and -> 0 for very negative x;
* BF16 rounding: hand-worked ties (to even, normal and subnormal) and
  agreement with the independent float32 -> BF16 rounding on every float32
  input drawn;
* SwiGLU with up = 1 and a gate where sigmoid rounds to 1 reduces to the
  plain 1x128 quantizer of the gate (catches swapped halves), and up = 0
  gives all-zero tiles with signed zero codes;
* the acceptance rule accepts the oracle's own output and rejects a planted
  error in a code or a scale.
"""

import math

import numpy as np
import pytest

from oracle import e4m3, moe, quantize as Q
import synth


def _bits(vals):
    return e4m3.f32_to_bf16_bits_rne(np.asarray(vals, dtype=np.float32))


def test_gather_hand_worked():
    codes = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12]], dtype=np.uint8)
    scales = np.array([[0.5], [0.25], [2.0]], dtype=np.float32)
    c, s = moe.gather_rows(codes, scales, np.array([2, 0, 2, 3, -1, 1], dtype=np.int32))
    assert c.tolist() == [[9, 10, 11, 12], [1, 2, 3, 4], [9, 10, 11, 12], [0, 0, 0, 0], [0, 0, 0, 0],
                          [5, 6, 7, 8]]
    assert s[:, 0].tolist() == [2.0, 0.5, 2.0, 0.0, 0.0, 0.25]


def test_gather_commutes_with_row_quantization():
    rng = np.random.default_rng(3)
    x = synth.bf16_rne((rng.standard_normal((50, 300)) * np.exp2(rng.integers(-4, 5, (50, 1)))).astype(np.float32))
    idx = rng.integers(0, 50, 80).astype(np.int32)
    for mode in (Q.FREE, Q.POW2):
        c, s = Q.quantize_rows(x, mode)
        gc, gs = moe.gather_rows(c, s, idx)
        wc, ws = Q.quantize_rows(x[idx], mode)
        assert np.array_equal(gc, wc) and np.array_equal(gs, ws)


def test_silu_closed_forms():
    assert moe.silu(0.0) == 0.0
    ln3 = math.log(3.0)
    assert moe.silu(ln3) == pytest.approx(0.75 * ln3, rel=1e-15)
    assert moe.silu(-ln3) == pytest.approx(-0.25 * ln3, rel=1e-15)
    x = np.random.default_rng(5).standard_normal(1000) * 5
    assert np.allclose(moe.silu(x) - moe.silu(-x), x, rtol=0, atol=1e-13)
    assert moe.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(moe.silu(-800.0)) < 1e-300


def test_bf16_rounding_ties_and_float32_agreement():
    hand = [(1 + 2.0 ** -8, 1.0), (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6), (1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -7),
            (-(1 + 2.0 ** -8), -1.0), (2.0 ** -134, 0.0), (3 * 2.0 ** -134, 2.0 ** -132),
            (2.0 ** -133, 2.0 ** -133), (255.5, 256.0), (254.5, 254.0)]
    for v, want in hand:
        assert moe.round_bf16(np.array([v]))[0] == want, v
    rng = np.random.default_rng(11)
    f = np.concatenate([rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000)),
                        rng.standard_normal(1000) * 2.0 ** -130]).astype(np.float32)
    assert np.array_equal(moe.bf16_bits(moe.round_bf16(f.astype(np.float64))), e4m3.f32_to_bf16_bits_rne(f))


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_swiglu_reduces_to_plain_quantizer(mode):
    rng = np.random.default_rng(7)
    gate = _bits(40.0 + rng.random((9, 260)) * 60.0)  # sigmoid(g) rounds to 1 in float64 x BF16
    up = _bits(np.ones((9, 260)))
    c, s = moe.swiglu_quantize(np.concatenate([gate, up], axis=1), mode)
    wc, ws = Q.quantize_rows(gate, mode)
    assert np.array_equal(c, wc) and np.array_equal(s, ws)
    # up = 0: zero tiles, scale 0, codes keep the sign of silu(g) * 0
    g2 = _bits(rng.standard_normal((3, 128)))
    c0, s0 = moe.swiglu_quantize(np.concatenate([g2, _bits(np.zeros((3, 128)))], axis=1), mode)
    assert np.all(s0 == 0)
    neg = e4m3.bf16_bits_to_f32(g2) < 0
    assert np.array_equal(c0, np.where(neg, 0x80, 0x00).astype(np.uint8))


def test_accept_rule():
    rng = np.random.default_rng(13)
    x = _bits(rng.standard_normal((40, 2 * 333)) * 3)
    for mode in (Q.FREE, Q.POW2):
        c, s = moe.swiglu_quantize(x, mode)
        assert moe.swiglu_accept(x, mode, c, s).all()
        bad = c.copy()
        bad[7, 130] ^= 0x01
        acc = moe.swiglu_accept(x, mode, bad, s)
        assert not acc[7, 1] and acc.sum() == acc.size - 1
        bad_s = s.copy()
        bad_s[2, 0] *= 2
        assert not moe.swiglu_accept(x, mode, c, bad_s)[2, 0]


def test_candidates_only_near_midpoints():
    """The second candidate differs from the rounded value only within the
    band around a midpoint, and is then the adjacent BF16 number."""
    rng = np.random.default_rng(17)
    x = _bits(rng.standard_normal((64, 2 * 512)) * 2)
    y = moe.swiglu_exact(x)
    c1, c2 = moe.swiglu_candidates(x)
    assert np.array_equal(c1, moe.round_bf16(y))
    diff = c1 != c2
    lo, hi, q = moe._bf16_grid(y)
    assert np.all(np.abs(c1[diff] - c2[diff]) == q[diff])
    mid = lo + q / 2
    assert np.all(np.abs(y[diff] - mid[diff]) <= moe.BAND_REL * np.abs(y[diff]) + moe.BAND_ABS)
    assert 0 < diff.sum() < 0.01 * diff.size
    # a midpoint between two BF16 numbers and its neighbours on the grid
    lo, hi, q = moe._bf16_grid(np.array([1 + 2.0 ** -8, -(1 + 2.0 ** -8)]))
    assert lo.tolist() == [1.0, -(1 + 2.0 ** -7)] and hi.tolist() == [1 + 2.0 ** -7, -1.0]


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _ulp_push(x32, k):
    """float32 values moved k ulps (k = -1, 0, 1) toward +inf / -inf."""
    x32 = np.asarray(x32, dtype=np.float32)
    if k > 0:
        return np.nextafter(x32, np.float32(np.inf))
    if k < 0:
        return np.nextafter(x32, np.float32(-np.inf))
    return x32


def _swiglu_f32(g, u, k_exp, k_rcp):
    """The GPU's float32 SwiGLU sequence, emulated step by step: the two-part
    log2(e) reduction with fused multiply-adds (exact products in float64,
    one rounding each), exp2 and the reciprocal correctly rounded and then
    pushed k ulps (the hardware's one-ulp accuracy), ldexp exact."""
    g = _f32(g)
    u = _f32(u)
    x = np.maximum(-np.abs(g), np.float32(-104.0))
    hi = np.float32(1.44269502162933349609375)
    lo = np.float32(1.92596298909109e-8)
    n = np.rint(_f32(x.astype(np.float64) * hi))
    f1 = _f32(x.astype(np.float64) * hi - n)
    f = _f32(x.astype(np.float64) * lo + f1)
    p = _ulp_push(_f32(np.exp2(f.astype(np.float64))), k_exp)
    t = _f32(np.ldexp(p.astype(np.float64), n.astype(np.int64)))
    r = _ulp_push(_f32(1.0 / _f32(1.0 + t.astype(np.float64)).astype(np.float64)), k_rcp)
    sg = np.where(g >= 0, r, _f32(t.astype(np.float64) * r))
    return _f32(_f32(g.astype(np.float64) * sg).astype(np.float64) * u)


def _swiglu_f32_direct(g, u, k_exp, k_rcp):
    """The GPU's float32 SwiGLU for gates >= -64, emulated step by step:
    g times c1 = 47274 / 2^15 (exact in float32 for a BF16 g; checked),
    exp2 correctly rounded and pushed k_exp ulps, the first-order factor
    1 - g * RN32(k) applied by one fused multiply-add, 1 + e, the reciprocal
    correctly rounded and pushed k_rcp ulps, then two products."""
    g = _f32(g)
    u = _f32(u)
    c1 = np.float32(47274.0 / 32768.0)
    k = np.float32(4.8884954e-06)
    arg64 = -g.astype(np.float64) * np.float64(c1)
    arg = _f32(arg64)
    assert np.array_equal(arg.astype(np.float64), arg64)  # the product is exact
    e1 = _ulp_push(_f32(np.exp2(arg.astype(np.float64))), k_exp)
    h = _f32(g.astype(np.float64) * np.float64(k))
    e = _f32(e1.astype(np.float64) - h.astype(np.float64) * e1.astype(np.float64))
    r = _ulp_push(_f32(1.0 / _f32(1.0 + e.astype(np.float64)).astype(np.float64)), k_rcp)
    return _f32(_f32(g.astype(np.float64) * r).astype(np.float64) * u)


def test_swiglu_direct_form_error_bound():
    """The bound of the form taken when every gate is at least -64
    (oracle.moe.swiglu_rel_error_bound_direct) against the emulation above
    on 200,000 BF16 pairs with gates over [-64, 64] and a dense core, the
    hardware exp2 and reciprocal pushed one ulp either way; the split
    constants are what they claim (c1 has 16 significant bits and is
    log2(e) to that precision, RN32(k) is the float32 rounding of
    1 - c1 ln 2), and the bound is inside the overall one and the band."""
    c1 = 47274.0 / 32768.0
    assert 47274 < 2 ** 16 and abs(c1 - 1 / np.log(2)) < 2.0 ** -16
    assert np.float32(4.8884954e-06) == np.float32(1.0 - c1 * np.log(2.0))
    bound = moe.swiglu_rel_error_bound_direct()
    assert bound <= moe.swiglu_rel_error_bound() < moe.BAND_REL / 2
    rng = np.random.default_rng(12)
    g = np.concatenate([rng.uniform(-64, 64, 150000), rng.uniform(-64, -40, 25000),
                        rng.standard_normal(25000) * 1.7]).astype(np.float32)
    ub = rng.standard_normal(g.size).astype(np.float32)
    gb = e4m3.bf16_bits_to_f32(_bits(g)).astype(np.float64)
    assert gb.min() >= -64
    uv = e4m3.bf16_bits_to_f32(_bits(ub)).astype(np.float64)
    exact = moe.silu(gb) * uv
    worst = 0.0
    for k_exp in (-1, 0, 1):
        for k_rcp in (-1, 0, 1):
            y = _swiglu_f32_direct(gb, uv, k_exp, k_rcp).astype(np.float64)
            err = np.abs(y - exact)
            ok = err <= bound * np.abs(exact) + moe.BAND_ABS
            assert ok.all(), (k_exp, k_rcp, gb[~ok][:3], (err / np.abs(exact))[~ok][:3])
            normal = np.abs(exact) > 2.0 ** -100
            worst = max(worst, float((err[normal] / np.abs(exact[normal])).max()))
    assert worst > bound / 8, (worst, bound)


def test_swiglu_error_bound_holds_and_sits_inside_the_band():
    """The composed bound of the general form
    (oracle.moe.swiglu_rel_error_bound_general) against an
    emulation of the kernel's float32 arithmetic on 200,000 BF16 (gate, up)
    pairs spread over gates in [-40, 40] (and tails to -104), with the
    hardware exp2 and reciprocal results pushed one ulp up or down: every
    emulated result is within the bound of the exact value, and the bound is
    inside the acceptance band BAND_REL."""
    bound = moe.swiglu_rel_error_bound_general()
    assert bound <= moe.swiglu_rel_error_bound() < moe.BAND_REL / 2
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.uniform(-40, 40, 150000), rng.uniform(-104, -40, 25000),
                        rng.standard_normal(25000) * 1.7]).astype(np.float32)
    ub = rng.standard_normal(g.size).astype(np.float32)
    gb = e4m3.bf16_bits_to_f32(_bits(g)).astype(np.float64)
    uv = e4m3.bf16_bits_to_f32(_bits(ub)).astype(np.float64)
    exact = moe.silu(gb) * uv
    worst = 0.0
    for k_exp in (-1, 0, 1):
        for k_rcp in (-1, 0, 1):
            y = _swiglu_f32(gb, uv, k_exp, k_rcp).astype(np.float64)
            err = np.abs(y - exact)
            ok = err <= bound * np.abs(exact) + moe.BAND_ABS
            assert ok.all(), (k_exp, k_rcp, gb[~ok][:3], (err / np.abs(exact))[~ok][:3])
            normal = np.abs(exact) > 2.0 ** -100
            worst = max(worst, float((err[normal] / np.abs(exact[normal])).max()))
    # the bound is not loose by orders of magnitude either
    assert worst > bound / 8, (worst, bound)
