"""Pins for the oracle's quantizers (CPU).

jp-study.kr doc 258368 ¶1 fixes online max-abs scaling per 1x128 activation
tile and per 128x128 weight block; tmdrlife.com wr_id=13334 ¶4 fixes
power-of-two scales for some activations.  What the pages and the arithmetic
then force, and what is checked here without re-deriving the oracle's own
formula:

* hand-worked tiles (tests/golden/quant_tiles.txt);
* the max-abs element of every nonzero tile lands on +-448 (code 0x7E/0xFE);
* dequantization error |x - dec(code) * s| <= 1/2 ulp_E4M3(x/s) * s plus one
  float32 rounding of the quotient (free scales), exactly 1/2 ulp for
  power-of-two scales;
* power-of-two scales are exact powers of two with amax / s in (224, 448];
* scaling a tile by 2^j scales s by 2^j and leaves the codes unchanged;
* negating a tile flips only the code sign bits;
* tiles are independent: concatenation, row gather and block locality;
* the token-axis variant equals per-column quantization, cross-checked with
  explicit per-column loops.
"""

from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import e4m3, quantize as Q
import synth


def _bits(vals):
    return e4m3.f32_to_bf16_bits_rne(np.asarray(vals, dtype=np.float32))


def test_hand_worked_tiles(golden):
    for row in golden("quant_tiles.txt"):
        name, mode, cols = row[0], row[1], int(row[2])
        scales_want = [int(s, 16) for s in row[3].split(",")]
        x = np.zeros((1, cols), dtype=np.float32)
        if name == "A":
            x[0, :] = 1.0
            x[0, 0] = 448.0
        elif name in "BC":
            x[0, :3] = [-2.0, 1.0, 0.5]
        elif name == "D":
            x[0, 0] = 1.875
        elif name == "E":
            x[0, 0] = 1.75
        elif name == "F":
            x[0, 0] = -0.0
        elif name == "G":
            x[0, 128:130] = [3.0, -1.5]
        codes, scales = Q.quantize_rows(_bits(x), mode)
        assert list(scales.reshape(-1).view(np.uint32)) == scales_want, name
        for item in row[4:]:
            c, idx = item.split("@")
            assert codes[0, int(idx)] == int(c, 16), (name, item, hex(codes[0, int(idx)]))


def _ulp_e4m3(q):
    q = np.abs(np.asarray(q, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    return np.where(q < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3))


def _tiles_rows(x_bits, codes, scales):
    """(x, dec, s) as float64 arrays aligned per element for 1x128 row tiles."""
    x = e4m3.bf16_bits_to_f64(x_bits)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)[:, : x.shape[1]]
    return x, e4m3.decode(codes), s


def _check_row_invariants(x_bits, mode):
    codes, scales = Q.quantize_rows(x_bits, mode)
    x, dec, s = _tiles_rows(x_bits, codes, scales)
    rows, cols = x.shape
    nb = scales.shape[1]
    # max element of each nonzero tile -> +-448
    for r in range(rows):
        for b in range(nb):
            seg = np.abs(x[r, b * 128:(b + 1) * 128])
            if seg.max() == 0:
                assert scales[r, b] == 0
                continue
            j = b * 128 + int(np.argmax(seg))
            assert abs(dec[r, j]) == 448.0 or mode == Q.POW2
            if mode == Q.POW2:
                ratio = Fraction(float(seg.max())) / Fraction(float(scales[r, b]))
                assert Fraction(224) < ratio <= Fraction(448)
                m, _ = np.frexp(scales[r, b])
                assert m == 0.5  # an exact power of two (incl. subnormal)
            else:
                # s is the float32 nearest amax/448: within half an ulp
                sf = Fraction(float(scales[r, b]))
                exact = Fraction(float(seg.max())) / 448
                ulp = Fraction(float(np.spacing(np.float32(scales[r, b]))))
                assert abs(sf - exact) <= ulp / 2
    nz = s > 0
    err = np.abs(x - dec * s)
    q = np.where(nz, x / np.where(nz, s, 1.0), 0.0)
    bound = 0.5 * _ulp_e4m3(q) * s
    if mode == Q.FREE:
        bound = bound + 2.0 ** -24 * np.abs(x)
    assert np.all(err[nz] <= bound[nz] * (1 + 1e-12))
    # zero tiles: codes are signed zeros matching the input sign
    zt = ~nz
    assert np.all((codes[zt] & 0x7F) == 0)
    assert np.array_equal(codes[zt] >> 7, (x_bits[zt] >> 15).astype(np.uint8))
    return codes, scales


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_invariants_tiny_linear(mode):
    d = synth.tiny_linear()
    _check_row_invariants(d["a"], mode)


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_invariants_student_t_ragged(mode):
    rng = np.random.default_rng(3)
    x = rng.standard_t(3, size=(6, 300)).astype(np.float32)
    x[2, 128:256] = 0.0
    x[3, 5] = -0.0
    x[3, :128] = 0.0
    x[3, 7] = -0.0
    _check_row_invariants(_bits(x), mode)


@settings(max_examples=40, deadline=None)
@given(rows=st.integers(1, 3), cols=st.integers(1, 300), seed=st.integers(0, 2**31 - 1),
       spread=st.integers(0, 40), mode=st.sampled_from([Q.FREE, Q.POW2]))
def test_invariants_property(rows, cols, seed, spread, mode):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-spread, spread + 1, (rows, cols)))
    x = x.astype(np.float32)
    x[rng.random((rows, cols)) < 0.05] = 0.0
    _check_row_invariants(_bits(x), mode)


@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_power_of_two_equivariance_and_negation(mode):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4, 256)) * 3).astype(np.float32)
    xb = _bits(x)
    c0, s0 = Q.quantize_rows(xb, mode)
    for j in (-20, -3, 1, 7, 30):
        xs = _bits(e4m3.bf16_bits_to_f32(xb) * np.float32(2.0 ** j))
        c1, s1 = Q.quantize_rows(xs, mode)
        assert np.array_equal(c0, c1), j
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32)), j
    cn, sn = Q.quantize_rows(xb ^ np.uint16(0x8000), mode)
    assert np.array_equal(sn, s0)
    assert np.array_equal(cn, c0 ^ np.uint8(0x80))


def test_tile_independence_concat_and_gather():
    rng = np.random.default_rng(9)
    x1 = _bits(rng.standard_normal((5, 256)))
    x2 = _bits(rng.standard_normal((5, 384)) * 100)
    c, s = Q.quantize_rows(np.concatenate([x1, x2], axis=1))
    c1, s1 = Q.quantize_rows(x1)
    c2, s2 = Q.quantize_rows(x2)
    assert np.array_equal(c, np.concatenate([c1, c2], axis=1))
    assert np.array_equal(s, np.concatenate([s1, s2], axis=1))
    # quantize-then-gather == gather-then-quantize (jp-study.kr doc 258368 ¶1:
    # activations are quantized before the MoE dispatch)
    idx = np.array([4, 0, 0, 3])
    cg, sg = Q.quantize_rows(x2[idx])
    assert np.array_equal(cg, c2[idx]) and np.array_equal(sg, s2[idx])


def test_token_axis_matches_column_loops():
    rng = np.random.default_rng(11)
    x = _bits(rng.standard_t(3, size=(300, 5)))
    codes_t, scales = Q.quantize_token_t(x)
    assert codes_t.shape == (5, 300) and scales.shape == (5, 3)
    xf = e4m3.bf16_bits_to_f32(x)
    for c in range(5):
        for b in range(3):
            col = xf[b * 128:(b + 1) * 128, c]
            amax = np.float32(np.max(np.abs(col)))
            s = np.float32(amax / np.float32(448))
            assert scales[c, b] == s
            want = e4m3.encode((col / s).astype(np.float32))
            assert np.array_equal(codes_t[c, b * 128:b * 128 + col.size], want)


def test_weight_blocks_locality_and_max():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((200, 300)) * 0.02).astype(np.float32)
    w[5, 7] = 3.0  # block (0, 0)
    wb = _bits(w)
    codes, scales = Q.quantize_blocks(wb)
    assert scales.shape == (2, 3)
    assert codes[5, 7] == 0x7E
    # every block's max element lands on 448, and changing one block leaves
    # the others untouched
    x = e4m3.bf16_bits_to_f64(wb)
    dec = e4m3.decode(codes)
    for bn in range(2):
        for bk in range(3):
            blk = np.abs(x[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128])
            i, j = np.unravel_index(np.argmax(blk), blk.shape)
            assert abs(dec[bn * 128 + i, bk * 128 + j]) == 448.0
    w2 = w.copy()
    w2[150, 290] = 50.0  # block (1, 2)
    codes2, scales2 = Q.quantize_blocks(_bits(w2))
    same = np.ones((2, 3), bool)
    same[1, 2] = False
    assert np.array_equal(scales2[same], scales[same])
    assert np.array_equal(codes2[:128], codes[:128])
    assert np.array_equal(codes2[128:, :256], codes[128:, :256])
    # a 128x128 block equals the 1x128 quantizer run on the block flattened:
    # both take one max over exactly the block's elements
    # the block scale comes from the max over all 128x128 elements
    blk = wb[:128, :128]
    amax = np.max(np.abs(e4m3.bf16_bits_to_f32(blk)))
    assert scales[0, 0] == np.float32(amax / np.float32(448))


def test_pow2_scale_range_edges():
    # amax exactly at 1.75 * 2^E and just above, incl. BF16 subnormals
    vals = [1.75, 1.7578125, 1.0, 1.9921875, 2.0 ** -130, 1.75 * 2.0 ** -127, 3.0 * 2.0 ** 100]
    for v in vals:
        x = np.zeros((1, 128), np.float32)
        x[0, 0] = v
        xb = _bits(x)
        amax = float(e4m3.bf16_bits_to_f32(xb)[0, 0])
        codes, s = Q.quantize_rows(xb, Q.POW2)
        ratio = Fraction(amax) / Fraction(float(s[0, 0]))
        assert Fraction(224) < ratio <= 448, v
        # q = x / s is exact, so the code is within half an E4M3 ulp of it
        dec = Fraction(float(e4m3.decode(codes)[0, 0]))
        assert abs(dec - ratio) <= Fraction(float(_ulp_e4m3(float(ratio)))) / 2, v


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (130, 300), (1, 129)])
@pytest.mark.parametrize("mode", [Q.FREE, Q.POW2])
def test_weight_blocks_commute_with_transpose(n, k, mode):
    """A square block's max-abs does not depend on orientation, so quantizing
    W^T per 128x128 block gives exactly the transpose of W quantized: the
    reading that lets the activation gradient reuse the weight blocks."""
    rng = np.random.default_rng(n * 7 + k)
    w = synth.bf16_rne((rng.standard_normal((n, k)) * np.exp2(rng.integers(-6, 6, (n, k)))).astype(np.float32))
    c, s = Q.quantize_blocks(w, mode)
    ct, st = Q.quantize_blocks(np.ascontiguousarray(w.T), mode)
    assert np.array_equal(ct, c.T)
    assert np.array_equal(st.view(np.uint32), s.T.view(np.uint32))
