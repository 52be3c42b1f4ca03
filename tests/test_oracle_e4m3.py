"""Pins for the oracle's E4M3 codec (CPU).

The codec follows the E4M3 definition (why-be.co.kr wr_id=35533 ¶2: 4-bit
exponent, 3-bit mantissa; OCP variant with max 448).  It is pinned against a
hand-typed code table, hand-worked roundings, torch's CPU float8_e4m3fn
implementation (an independent library), and a brute-force nearest-value
search in exact rational arithmetic.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_hand_table(golden):
    for code_s, val_s in golden("e4m3_codes.txt"):
        code = int(code_s, 16)
        got = e4m3.decode(np.array([code], dtype=np.uint8))[0]
        if val_s == "nan":
            assert math.isnan(got), hex(code)
        else:
            want = float(Fraction(val_s))
            assert got == want, (hex(code), got, want)
            assert math.copysign(1.0, got) == (-1.0 if val_s.startswith("-") else 1.0)


def test_decode_all_codes_match_torch():
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.nanmax(ours) == 448.0 and np.nanmin(np.abs(ours[ours != 0])) == 2.0 ** -9
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]


def test_decode_int_is_value_times_512():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3.decode_int(codes) * 2.0 ** -9, e4m3.decode(codes))
    with pytest.raises(ValueError):
        e4m3.decode_int(np.array([0x7F], dtype=np.uint8))


def test_encode_hand_worked(golden):
    for row in golden("e4m3_encode.txt"):
        val = np.float32(float(Fraction(row[0])) if row[0] != "-0.0" else -0.0)
        want = int(row[1], 16)
        got = int(e4m3.encode(np.array([val]))[0])
        assert got == want, (row, hex(got))


def _torch_encode(x):
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


LIMIT_BITS = int(np.array([464.0], dtype=np.float32).view(np.uint32)[0])


BAND_LO_BITS = int(np.array([2.0 ** -11], dtype=np.float32).view(np.uint32)[0])


@pytest.mark.slow
def test_encode_exhaustive_positive_vs_torch():
    """Every positive float32 bit pattern in [2^-11, 464] (torch gives NaN above 464).

    Below 2^-11 every value is closer to 0 than to 2^-9; those binades are
    covered on a stride, and their result is checked to be the zero code.
    """
    step = 1 << 24
    for lo in range(BAND_LO_BITS, LIMIT_BITS + 1, step):
        hi = min(lo + step, LIMIT_BITS + 1)
        x = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
        ours = e4m3.encode(x)
        ref = _torch_encode(x)
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (hex(lo + int(bad[0])), ours[bad[0]], ref[bad[0]])
    x = np.arange(0, BAND_LO_BITS, 101, dtype=np.uint32).view(np.float32)
    ours = e4m3.encode(x)
    assert np.array_equal(ours, _torch_encode(x)) and not ours.any()


def test_encode_negative_stride_vs_torch():
    """Negative patterns on a stride (sign handling and -0), plus all of [-2^-5, 0]."""
    pats = np.arange(0, LIMIT_BITS + 1, 977, dtype=np.uint32)
    small = np.arange(0, int(np.array([2.0 ** -5], np.float32).view(np.uint32)[0]), 13, dtype=np.uint32)
    for p in (pats, small):
        x = (p | np.uint32(0x80000000)).view(np.float32)
        assert np.array_equal(e4m3.encode(x), _torch_encode(x))


def _nearest_bruteforce(v):
    """Nearest finite E4M3 code by exhaustive search, ties to the even code."""
    best = None
    target = Fraction(abs(float(v)))
    for code in range(0x7F):  # finite non-negative codes 0x00..0x7E
        val = Fraction(float(e4m3.decode(np.array([code], np.uint8))[0]))
        d = abs(target - val)
        key = (d, code & 1)
        if best is None or key < best[0]:
            best = (key, code)
    code = best[1]
    if np.signbit(v):
        code |= 0x80
    return code


def test_encode_vs_bruteforce_nearest():
    rng = np.random.default_rng(1234)
    mags = np.exp2(rng.uniform(-14, 9, size=600)).astype(np.float32)
    mags = np.concatenate([mags, rng.integers(0, 900, 100).astype(np.float32) / np.float32(2)])
    signs = rng.choice([-1.0, 1.0], size=mags.size).astype(np.float32)
    vals = mags * signs
    ours = e4m3.encode(vals)
    for v, c in zip(vals, ours):
        if abs(float(v)) <= 464.0:
            assert int(c) == _nearest_bruteforce(v), (float(v), hex(int(c)))


def test_bf16_helpers_match_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(10000) * np.exp2(rng.uniform(-30, 30, 10000))).astype(np.float32)
    ours = e4m3.f32_to_bf16_bits_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = e4m3.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy())
