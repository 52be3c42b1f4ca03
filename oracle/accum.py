"""Accumulation emulators for the promotion-interval report -- oracle.

why-be.co.kr wr_id=35533 ¶4: inside the matrix unit the running sum is kept
in a limited bit width.  tmdrlife.com wr_id=13334 ¶2: on Hopper the FP8 GEMM
accumulates in fixed point, aligning the mantissa products by right-shifting
them to the largest exponent before adding.  jp-study.kr doc 258368 ¶3:
promoting the partial sum to FP32 every 128 elements of K is the smallest
interval that markedly improves precision.  The pages give no bit width.

``accumulate`` models one output element as a sequence of products summed in
intervals: inside an interval the sum is held in a W-bit fixed-point
accumulator aligned to the running maximum exponent (W=None: a float32
accumulator); at the end of each interval the partial is added to a float32
register ("promotion").  interval = len(terms) means no promotion.

Readings taken where the pages are silent: the alignment truncates toward
zero, both the accumulator and the incoming product are put on the grid
2^(E-W+1) of the larger exponent E before the exact addition; products enter
as float64 values of the dequantized operands.  The float32 steps are emulated through
float64 followed by a float32 cast.

Parity: pinned only in its closed-form special cases (W large equals the
exact sum; a product below the accumulator's grid is dropped; W=None with
interval 1 equals sequential float32 addition).  Beyond those the fixed-point
model is "parity unpinned": the pages fix neither the width nor the rounding.
"""

import numpy as np


def _fixed_add(acc, term, width):
    """acc + term in a width-bit accumulator aligned to the larger exponent."""
    mag = np.maximum(np.abs(acc), np.abs(term))
    _, e = np.frexp(mag)  # mag = f * 2^e, f in [0.5, 1): floor(log2 mag) = e - 1
    q = np.ldexp(1.0, (e - 1) - width + 1)
    q = np.where(mag == 0, 1.0, q)
    return np.trunc(acc / q) * q + np.trunc(term / q) * q


def accumulate(terms, interval, width=None):
    """Sum each row of ``terms`` (float64 [S, T]) as described above.

    Returns float64 [S] (values that are float32-representable).
    """
    terms = np.asarray(terms, dtype=np.float64)
    s_count, t_count = terms.shape
    out = np.zeros(s_count, dtype=np.float32)
    for start in range(0, t_count, interval):
        part = np.zeros(s_count, dtype=np.float64)
        for t in range(start, min(start + interval, t_count)):
            if width is None:
                part = (part + terms[:, t]).astype(np.float32).astype(np.float64)
            else:
                part = _fixed_add(part, terms[:, t], width)
        out = (out.astype(np.float64) + part.astype(np.float32)).astype(np.float32)
    return out.astype(np.float64)


def dequantize(codes_rows, scales_rows):
    """Values q*s (float64 [S, K]) of code rows with one scale per
    128-element block (scales_rows [S, K/128])."""
    from .e4m3 import decode
    return decode(codes_rows) * np.repeat(np.asarray(scales_rows, np.float64), 128, axis=1)


def dequantized_products(a_codes_rows, a_scales_rows, b_codes_rows, b_scales_rows):
    """Products (qa*sa)(qb*sb) along K for paired rows (float64 [S, K]).

    a_scales_rows / b_scales_rows are per 128-element block ([S, K/128]).
    """
    return dequantize(a_codes_rows, a_scales_rows) * dequantize(b_codes_rows, b_scales_rows)
