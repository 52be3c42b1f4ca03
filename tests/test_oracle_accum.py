"""Pins for the accumulation emulators (CPU) -- closed-form special cases only.

The emulators model the limited-width accumulation (why-be.co.kr wr_id=35533
¶4; tmdrlife.com wr_id=13334 ¶2) and promotion every 128 elements
(jp-study.kr doc 258368 ¶3).  The pages fix no accumulator width, so beyond
these cases the fixed-point model is parity unpinned.
"""

import numpy as np

from oracle import accum


def test_wide_accumulator_is_exact():
    rng = np.random.default_rng(0)
    terms = rng.integers(-1000, 1000, (16, 300)).astype(np.float64) * 2.0 ** -9
    got = accum.accumulate(terms, interval=300, width=60)
    assert np.array_equal(got, terms.sum(axis=1).astype(np.float32).astype(np.float64))


def test_small_term_below_grid_is_dropped():
    terms = np.array([[1.0, 2.0 ** -30, 2.0 ** -30]])
    assert accum.accumulate(terms, interval=3, width=24)[0] == 1.0
    # with promotion after every element the float32 register keeps nothing
    # either (2^-30 is below half an ulp of 1.0 in float32)
    assert accum.accumulate(terms, interval=1, width=None)[0] == 1.0
    # a term exactly on the grid survives
    terms = np.array([[1.0, 2.0 ** -23]])
    assert accum.accumulate(terms, interval=2, width=24)[0] == 1.0 + 2.0 ** -23


def test_float32_sequential_special_case():
    rng = np.random.default_rng(1)
    terms = rng.standard_normal((8, 50)).astype(np.float32).astype(np.float64)
    got = accum.accumulate(terms, interval=1, width=None)
    acc = np.zeros(8, np.float32)
    for t in range(50):
        acc = acc + terms[:, t].astype(np.float32)
    assert np.array_equal(got, acc.astype(np.float64))


def test_truncation_toward_zero_alignment():
    # acc = 1.5 (exp 0), term = -0.75 - 2^-25 with W = 24: the term is cut to
    # the 2^-23 grid toward zero -> -0.75, so the sum is exactly 0.75
    terms = np.array([[1.5, -0.75 - 2.0 ** -25]])
    assert accum.accumulate(terms, interval=2, width=24)[0] == 0.75


# ---- the FP8 matrix-core model (mfma_partials): closed-form cases --------

def _codes(vals):
    """E4M3 codes of exactly representable values (via the oracle encoder)."""
    from oracle import e4m3
    return e4m3.encode(np.asarray(vals, dtype=np.float32))


def _pair(a_vals, b_vals):
    a = np.zeros((1, 128), np.uint8)
    b = np.zeros((1, 128), np.uint8)
    a[0, :len(a_vals)] = _codes(a_vals)
    b[0, :len(b_vals)] = _codes(b_vals)
    return a, b


def test_mfma_model_single_products_are_exact():
    # one nonzero product per group of 8: every product sits on its own grid
    rng = np.random.default_rng(5)
    a = np.zeros((4, 128), np.uint8)
    b = np.zeros((4, 128), np.uint8)
    a[:, ::8] = rng.integers(1, 0x7E, (4, 16))
    b[:, ::8] = rng.integers(1, 0x7E, (4, 16))
    from oracle import e4m3
    exact = (e4m3.decode(a) * e4m3.decode(b)).sum(axis=1)
    p, t = accum.mfma_partials(a, b)
    assert np.array_equal(p[:, 0], exact)
    assert np.array_equal(t[:, 0], np.abs(e4m3.decode(a) * e4m3.decode(b)).sum(axis=1))


def test_mfma_model_grid_follows_exponent_sum():
    # group max (1.875*16)^2 = 900 has exponent sum 8 -> grid 2^-5, the same
    # grid as for 16*16 = 256; a second product 2.234375 (1.625*1.375) is cut
    # to 2.21875 in both groups
    a, b = _pair([30.0, 1.625, 0, 0, 0, 0, 0, 0, 16.0, 1.625], [30.0, 1.375, 0, 0, 0, 0, 0, 0, 16.0, 1.375])
    p, _ = accum.mfma_partials(a, b)
    assert p[0, 0] == (900.0 + 2.21875) + (256.0 + 2.21875)


def test_mfma_model_products_below_grid_vanish_and_truncate_toward_zero():
    # 2^8 * 2^8 sets grid 2^3 for its group; 1.875 * 2^5 = 60 -> 56, -60 -> -56,
    # 1.0 -> 0; the same values in the next group (no large product) are exact
    a, b = _pair([256.0, 60.0, -60.0, 1.0, 0, 0, 0, 0, 60.0, 1.0],
                 [256.0, 1.0, 1.0, 1.0, 0, 0, 0, 0, 1.0, 1.0])
    p, _ = accum.mfma_partials(a, b)
    assert p[0, 0] == 65536.0 + 56.0 - 56.0 + 0.0 + 60.0 + 1.0


def test_mfma_model_subnormal_operand_exponent():
    # a = 7*2^-9 (subnormal: exponent -6), w = 448 (exponent 8): sum 2 ->
    # grid 2^-11; a small product 71.5 grid steps wide keeps 71 of them
    small_a, small_b = 1.625 * 2.0 ** -3, 1.375 * 2.0 ** -3   # product 2.234375 * 2^-6
    a, b = _pair([7 * 2.0 ** -9, small_a], [448.0, small_b])
    p, _ = accum.mfma_partials(a, b)
    assert p[0, 0] == 7 * 2.0 ** -9 * 448.0 + 71 * 2.0 ** -11
