"""Pins for the oracle's block-scaled GEMMs and acceptance rule (CPU).

The GEMM definition (tmdrlife.com wr_id=13334 ¶3, jp-study.kr doc 258368 ¶3:
partials scaled and added in FP32 every 128 elements of K) is pinned by:

* hand-computed cases (tests/golden/gemm_small.txt);
* exact brute force on the tiny-linear shape: per-block dot products in
  int64 and the scale fold in exact rationals, versus the float64 oracle;
* closed forms: constant operands, selector weights, zero scales;
* cross-identities: grouped == per-group dense, Wgrad == dense when the
  per-row weight scales are constant over 128-row blocks, sampled
  evaluation == full evaluation;
* the acceptance rule on hand-made FP32 and BF16 cases.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm as G, quantize as Q
import synth


def _fr(x):
    return Fraction(float(x))


def test_hand_computed(golden):
    rows = {int(r[0]): (float(Fraction(r[1])), float(Fraction(r[2]))) for r in golden("gemm_small.txt")}
    # case 1
    a = np.full((1, 128), 0x38, np.uint8)
    w = np.full((1, 128), 0x40, np.uint8)
    c, s = G.gemm(a, np.array([[0.5]], np.float32), w, np.array([[0.25]], np.float32))
    assert (c[0, 0], s[0, 0]) == rows[1]
    # case 2
    a = np.full((1, 256), 0x38, np.uint8)
    w = np.full((1, 256), 0x38, np.uint8)
    w[0, 128:] = 0xB8
    c, s = G.gemm(a, np.array([[1.0, 2.0]], np.float32), w, np.array([[1.0, 0.5]], np.float32))
    assert (c[0, 0], s[0, 0]) == rows[2]
    # case 3
    a = np.zeros((1, 128), np.uint8)
    a[0, 0], a[0, 1] = 0x7E, 0x01
    w = np.zeros((1, 128), np.uint8)
    w[0, :2] = 0x7E
    c, s = G.gemm(a, np.ones((1, 1), np.float32), w, np.ones((1, 1), np.float32))
    assert (c[0, 0], s[0, 0]) == rows[3]


def _tiny_quantized():
    d = synth.tiny_linear()
    a_c, a_s = Q.quantize_rows(d["a"])
    w_c, w_s = Q.quantize_blocks(d["w"])
    return a_c, a_s, w_c, w_s


def test_exact_bruteforce_tiny_linear():
    a_c, a_s, w_c, w_s = _tiny_quantized()
    c, s = G.gemm(a_c, a_s, w_c, w_s)
    ia = e4m3.decode_int(a_c)  # int64, value = n * 2^-9
    iw = e4m3.decode_int(w_c)
    m, k = a_c.shape
    n = w_c.shape[0]
    nb = k // 128
    # integer per-block dots (exact), einsum over int64
    pint = np.einsum("mbk,nbk->mnb", ia.reshape(m, nb, 128), iw.reshape(n, nb, 128))
    rng = np.random.default_rng(0)
    picks = list(zip(rng.integers(0, m, 400), rng.integers(0, n, 400))) + [(0, 0), (m - 1, n - 1)]
    for i, j in picks:
        exact = sum(_fr(a_s[i, b]) * _fr(w_s[j // 128, b]) * Fraction(int(pint[i, j, b]), 2 ** 18)
                    for b in range(nb))
        assert abs(Fraction(float(c[i, j])) - exact) <= Fraction(float(s[i, j])) * Fraction(1, 2 ** 48)


def test_constant_operands_closed_form():
    for ca, cw in [(0x38, 0x40), (0x7E, 0xFE), (0x01, 0x44), (0x33, 0x2A)]:
        k = 512
        a = np.full((3, k), ca, np.uint8)
        w = np.full((130, k), cw, np.uint8)
        sa = np.full((3, k // 128), 0.37, np.float32)
        sw = np.full((2, k // 128), 1.9e-3, np.float32)
        c, s = G.gemm(a, sa, w, sw)
        va, vw = e4m3.decode(np.array([ca, cw], np.uint8))
        want = k * va * vw * float(np.float32(0.37)) * float(np.float32(1.9e-3))
        assert np.allclose(c, want, rtol=1e-15, atol=0)
        assert np.allclose(s, abs(want), rtol=1e-15, atol=0)


def test_selector_weights_exact():
    rng = np.random.default_rng(2)
    m, n, k = 4, 256, 384
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    sa = rng.uniform(0.01, 2, (m, k // 128)).astype(np.float32)
    w = np.zeros((n, k), np.uint8)
    pos = rng.integers(0, 128, (n, k // 128))
    sgn = rng.integers(0, 2, (n, k // 128))
    for j in range(n):
        for b in range(k // 128):
            w[j, b * 128 + pos[j, b]] = 0x38 | (0x80 * sgn[j, b])
    sw = rng.uniform(0.01, 2, (2, k // 128)).astype(np.float32)
    c, _ = G.gemm(a, sa, w, sw)
    va = e4m3.decode(a)
    for i in range(m):
        for j in range(0, n, 17):
            want = sum(_fr(sa[i, b]) * _fr(sw[j // 128, b]) * _fr(va[i, b * 128 + pos[j, b]])
                       * (-1 if sgn[j, b] else 1) for b in range(k // 128))
            assert abs(_fr(c[i, j]) - want) <= abs(want) * Fraction(1, 2 ** 50)


def test_zero_scales_contribute_nothing():
    a_c, a_s, w_c, w_s = _tiny_quantized()
    a_s = a_s.copy()
    a_s[5, :] = 0
    a_s[7, 2] = 0
    c, s = G.gemm(a_c, a_s, w_c, w_s)
    assert not c[5].any() and not s[5].any()
    a_c2 = a_c.copy()
    a_c2[7, 256:384] = 0x55  # garbage under a zero scale changes nothing
    c2, _ = G.gemm(a_c2, a_s, w_c, w_s)
    assert np.array_equal(c2[7], c[7])


def test_grouped_equals_per_group_dense():
    rng = np.random.default_rng(4)
    k, n = 256, 160
    offsets = np.array([0, 3, 3, 10, 11], np.int32)  # one empty group
    rows = 12  # last row covered by no group
    a = rng.integers(0, 0x7E, (rows, k)).astype(np.uint8)
    sa = rng.uniform(0.1, 1, (rows, 2)).astype(np.float32)
    w = rng.integers(0, 0x7E, (4, n, k)).astype(np.uint8) | (rng.integers(0, 2, (4, n, k)) * 0x80).astype(np.uint8)
    sw = rng.uniform(0.1, 1, (4, 2, 2)).astype(np.float32)
    c, s = G.grouped_gemm(a, sa, offsets, w, sw)
    for g in range(4):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            cg, sg = G.gemm(a[lo:hi], sa[lo:hi], w[g], sw[g])
            assert np.array_equal(c[lo:hi], cg) and np.array_equal(s[lo:hi], sg)
    assert np.isnan(c[11]).all()


def test_wgrad_equals_dense_with_blockwise_constant_scales():
    rng = np.random.default_rng(6)
    nout, kin, t = 20, 256, 384
    dy = rng.integers(0, 0x7E, (nout, t)).astype(np.uint8)
    xt = (rng.integers(0, 0x7E, (kin, t)) | (rng.integers(0, 2, (kin, t)) * 0x80)).astype(np.uint8)
    sdy = rng.uniform(0.1, 1, (nout, 3)).astype(np.float32)
    blocks = rng.uniform(0.1, 1, (2, 3)).astype(np.float32)
    sx = np.repeat(blocks, 128, axis=0)  # per-row scales, constant per 128 rows
    c1, s1 = G.wgrad(dy, sdy, xt, sx)
    c2, s2 = G.gemm(dy, sdy, xt, blocks)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_sampled_evaluation_matches_full():
    a_c, a_s, w_c, w_s = _tiny_quantized()
    c, s = G.gemm(a_c, a_s, w_c, w_s)
    rows = np.array([0, 5, 127, 64])
    cols = np.array([255, 0, 128, 129])
    ca, sa = G.gemm_at(a_c, a_s, w_c, w_s, rows, cols)
    assert np.allclose(ca, c[rows, cols], rtol=1e-14, atol=0)
    assert np.allclose(sa, s[rows, cols], rtol=1e-14, atol=0)
    # per-row weight scales (Wgrad form)
    w_row_s = np.repeat(w_s, 128, axis=0)
    cw, _ = G.gemm_at(a_c, a_s, w_c, w_row_s, rows, cols, w_block_rows=False)
    assert np.allclose(cw, c[rows, cols], rtol=1e-14, atol=0)


def test_acceptance_rule_f32_and_bf16():
    c_ref = np.array([1.0, 1.0, 1.00390625, 100.0])
    s_ref = np.array([0.0, 0.0, 0.0, 1000.0])  # tol: 1e-6, 1e-6, 1e-6, 0.010001
    ok = G.accept_f32(np.array([1.0 + 9e-7, 1.0 + 2e-6, 1.00390625, 100.01]), c_ref, s_ref)
    assert list(ok) == [True, False, True, True]
    bf = lambda v: e4m3.f32_to_bf16_bits_rne(np.array(v, np.float32))
    # 1.0 with tiny tolerance: only 1.0 itself
    assert list(G.accept_bf16(bf([1.0, 1.0078125]), c_ref[:2], s_ref[:2])) == [True, False]
    # the exact midpoint of 1.0 and 1.0078125: both neighbours are roundings of
    # float32 values within 1e-6
    mid = np.array([1.00390625, 1.00390625])
    assert list(G.accept_bf16(bf([1.0, 1.0078125]), mid, np.zeros(2))) == [True, True]
    # 100 +- 0.01: the BF16 neighbours of 100 are 99.5 and 100.5 -> only 100
    assert list(G.accept_bf16(bf([100.0, 100.5, 99.5]), np.full(3, 100.0), np.full(3, 1000.0))) == [True, False, False]


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_acceptance_rule_quantized_output(mode):
    """The quantization of the exact result rounded to BF16 passes; a code
    moved by one step where the tolerance cannot reach, or a doubled scale,
    does not; so does the quantization of a BF16 result nudged within
    tolerance."""
    rng = np.random.default_rng(23)
    a = synth.bf16_rne(rng.standard_normal((40, 256)).astype(np.float32))
    w = synth.bf16_rne((rng.standard_normal((300, 256)) * 0.02).astype(np.float32))
    ac, as_ = Q.quantize_rows(a)
    wc, ws = Q.quantize_blocks(w)
    c, s = G.gemm(ac, as_, wc, ws)
    cb = e4m3.f32_to_bf16_bits_rne(c.astype(np.float32))
    codes, scales = Q.quantize_rows(cb, mode)
    ok = G.accept_quantized(codes, scales, c, s, mode)
    assert ok.shape == (40, 3) and ok.all()
    # a code two E4M3 steps away from the right one, on a large element
    bad = codes.copy()
    r, j = 5, int(np.argmax(np.abs(c[5, :128])))
    bad[r, j] = (int(bad[r, j]) & 0x80) | ((int(bad[r, j]) & 0x7F) - 2)
    acc = G.accept_quantized(bad, scales, c, s, mode)
    assert not acc[r, 0] and acc.sum() == acc.size - 1
    bad_s = scales.copy()
    bad_s[7, 2] *= 2
    assert not G.accept_quantized(codes, bad_s, c, s, mode)[7, 2]
    # a BF16 result inside the tolerance (one float32 step away) quantizes to
    # an accepted tile
    nudged = np.nextafter(c.astype(np.float32), np.float32(np.inf))
    codes2, scales2 = Q.quantize_rows(e4m3.f32_to_bf16_bits_rne(nudged), mode)
    assert G.accept_quantized(codes2, scales2, c, s, mode).all()


def test_block_spread_inputs_expose_misplaced_scales():
    """The scale-staging GPU cases (tests/test_gpu_scale_groups.py) feed tiles
    and blocks whose magnitudes differ by up to 2^24: taking any one row's
    scale from a neighbouring K block, a neighbouring row of the same 16-row
    group, or the next group, moves outputs outside the tolerance."""
    from tests.test_gpu_scale_groups import _block_spread, _tile_spread
    rng = np.random.default_rng(106)
    m, n, k = 64, 130, 128 * 6
    a_c, a_s = Q.quantize_rows(_tile_spread(rng, m, k))
    w_c, w_s = Q.quantize_blocks(_block_spread(rng, n, k))
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    def fails(a_s_bad, w_s_bad=w_s):
        bad, _ = G.gemm(a_c, a_s_bad, w_c, w_s_bad)
        return not G.accept_f32(bad, ref, s).all()
    swap_block = a_s.copy(); swap_block[5, [1, 2]] = a_s[5, [2, 1]]    # blocks 1 and 2 of row 5
    swap_group = a_s.copy(); swap_group[9, [3, 4]] = a_s[9, [4, 3]]    # last of group 0, first of group 1
    swap_row = a_s.copy(); swap_row[[16, 17], 0] = a_s[[17, 16], 0]     # two rows of one 16-row quarter
    swap_w = w_s.copy(); swap_w[1, [0, 4]] = w_s[1, [4, 0]]              # W block column 1, blocks 0 and 4
    assert fails(swap_block) and fails(swap_group) and fails(swap_row) and fails(a_s, swap_w)


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_scale_attained_against_brute_force(mode):
    """The scales of all 32,640 non-negative finite BF16 values, enumerated,
    against the closed-form membership test: every attained scale is
    recognised, and float32 values next to them (or random ones) are
    recognised exactly when they are in the enumerated set."""
    v = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    attained = Q._tile_scale(v, mode)
    assert G._scale_attained(attained, mode).all()
    table = set(attained.view(np.uint32).tolist())
    rng = np.random.default_rng(8)
    probe = np.concatenate([np.nextafter(attained, np.float32(np.inf)),
                            np.nextafter(attained, np.float32(0)),
                            rng.integers(0, 0x7F7FFFFF, 200000).astype(np.uint32).view(np.float32)])
    want = np.array([b in table for b in probe.view(np.uint32).tolist()])
    assert np.array_equal(G._scale_attained(probe, mode), want)


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_acceptance_rule_quantized_degenerate_tile(mode):
    """A tile whose exact results are all zero but whose tolerance is wide
    (S = 1000: every element may be any BF16 value in [-0.01, 0.01]): the
    quantization of any BF16 tensor inside that band is accepted, whatever
    its max-abs; a scale above the band's, or one that no BF16 max-abs
    yields, is rejected.  (Every code is admissible here: any value up to
    448 * s lies inside the band.)"""
    c = np.zeros((3, 128))
    s = np.full((3, 128), 1000.0)
    rng = np.random.default_rng(4)
    rows = []
    for top in (0.0078125, 2.0 ** -12, 0.009):  # max-abs of each row (BF16 values)
        x = rng.uniform(-top, top, 128).astype(np.float32)
        x[17] = top
        rows.append(e4m3.f32_to_bf16_bits_rne(x))
    bits = np.stack(rows)
    codes, scales = Q.quantize_rows(bits, mode)
    assert G.accept_quantized(codes, scales, c, s, mode).all()
    high = scales.copy()
    high[0, 0] = Q._tile_scale(np.float32(0.05), mode)
    assert not G.accept_quantized(codes, high, c, s, mode)[0, 0]
    if mode == Q.FREE:
        odd = scales.copy()
        odd[1, 0] = np.nextafter(scales[1, 0], np.float32(1))  # not RN32(v/448) of any BF16 v
        assert not G._scale_attained(odd[1:2, 0], mode)[0]
        assert not G.accept_quantized(codes, odd, c, s, mode)[1, 0]
