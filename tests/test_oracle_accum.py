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


def test_dequantized_products_hand_values():
    # E4M3: 0x38 = 1.0, 0x01 = 2^-9 (smallest subnormal), 0xC4 = -3.0,
    # 0x7E = 448; one scale per 128-element block
    a = np.zeros((1, 256), np.uint8)
    b = np.zeros((1, 256), np.uint8)
    a[0, :4] = [0x38, 0x01, 0xC4, 0x7E]
    b[0, :4] = [0x38, 0x38, 0x38, 0x01]
    a[0, 128] = 0x38
    b[0, 128] = 0xC4
    sa = np.array([[0.5, 4.0]], np.float32)
    sb = np.array([[2.0, 0.25]], np.float32)
    da = accum.dequantize(a, sa)
    assert da[0, :4].tolist() == [0.5, 2.0 ** -10, -1.5, 224.0] and da[0, 128] == 4.0
    p = accum.dequantized_products(a, sa, b, sb)
    assert p[0, :4].tolist() == [1.0, 2.0 ** -9, -3.0, 224.0 * 2.0 ** -8] and p[0, 128] == -3.0
    assert not p[0, 4:128].any() and not p[0, 129:].any()
