"""E4M3 (OCP "E4M3FN") codec and BF16 helpers -- oracle, test infrastructure.

why-be.co.kr wr_id=35533 ¶2: every GEMM tensor (Fprop, Dgrad, Wgrad) is held
in E4M3, a format with a 4-bit exponent and a 3-bit mantissa.  The pages name
the bit split only; the variant taken is the OCP one without infinities:

* exponent bias 7, so the smallest normal is 2^-6;
* exponent field 0 holds subnormals n * 2^-9, n = 1..7;
* the all-ones pattern S.1111.111 is NaN; S.1111.110 = 448 is the largest
  finite value; there is no infinity.

``encode`` rounds to nearest, ties to even mantissa, saturates finite values
above 448 to 448 and keeps the sign of zero.  It works on the float32 bit
pattern with integer arithmetic only, so no library cast is involved.

Pins (tests/test_oracle_e4m3.py): the 256 decoded values against the format
table typed by hand in tests/golden/e4m3_codes.txt and against torch's CPU
``float8_e4m3fn`` view; ``encode`` against torch's CPU cast for every
positive float32 below 464 (exhaustive) and for samples of negatives; and
against a brute-force nearest-value search over the 127 finite magnitudes.
"""

import numpy as np

MAX_FINITE = 448.0
CODE_MAX = 0x7E
CODE_NAN = 0x7F


def decode(codes):
    """E4M3 codes (uint8 array) -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man.astype(np.float64) * 2.0 ** -9
    nor = (8 + man).astype(np.float64) * np.exp2(exp.astype(np.float64) - 10.0)
    val = np.where(exp == 0, sub, nor)
    val = np.where((c & 0x7F) == CODE_NAN, np.nan, val)
    return sign * val


def decode_int(codes):
    """E4M3 codes -> the integer n with value = n * 2^-9 (int64).

    Every finite E4M3 value is an integer multiple of 2^-9 (the subnormal
    step); |n| <= 448 * 2^9 = 229376 < 2^18.  NaN codes are rejected.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    if np.any((c & 0x7F) == CODE_NAN):
        raise ValueError("NaN code in operand")
    exp = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(exp == 0, man, (8 + man) << np.maximum(exp - 1, 0))
    return np.where(c & 0x80, -mag, mag)


def _rne_shift(v, s):
    """Round-to-nearest-even of v / 2^s for int64 v >= 0 and int64 s >= 1."""
    s = np.minimum(s, 40)  # v < 2^24, so any shift above 25 yields 0
    q = v >> s
    r = v & ((np.int64(1) << s) - 1)
    half = np.int64(1) << (s - 1)
    up = (r > half) | ((r == half) & ((q & 1) == 1))
    return q + up.astype(np.int64)


def encode(x):
    """float32 array -> E4M3 codes (uint8), RNE, saturating, signed zero.

    With |a| = sig * 2^ex exactly (sig the 24-bit significand of the float32
    pattern, ex its unbiased exponent minus 23):

    * below the smallest normal (|a| < 2^-6) the code is n = RNE(|a| * 2^9),
      n in [0, 8]; n = 8 lands on the smallest normal code 0x08 by itself;
    * otherwise, with e = floor(log2 |a|), n = RNE(|a| * 2^(3-e)) in [8, 16];
      n = 16 carries into the exponent (e += 1, n = 8); the code is
      ((e + 7) << 3) | (n - 8), saturated to 0x7E above 448;
    * the sign bit is copied, so a negative value that rounds to zero
      gives 0x80.
    NaN inputs give 0x7F | sign (inputs are required to be finite).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) & 1
    biased = (bits >> 23) & 0xFF
    frac = bits & 0x7FFFFF
    normal = biased > 0
    sig = np.where(normal, frac | 0x800000, frac)
    ex = np.where(normal, biased - 150, -149)  # |a| = sig * 2^ex

    # Subnormal-E4M3 branch: n = RNE(sig * 2^(ex + 9)); ex + 9 <= -15 here.
    n_sub = _rne_shift(sig, np.maximum(-(ex + 9), 1))
    # Normal-E4M3 branch: e = biased - 127, n = RNE(sig * 2^(ex + 3 - e)) and
    # ex + 3 - e = -20 for every normal float32.
    e = biased - 127
    n_nor = _rne_shift(sig, np.full_like(sig, 20))
    carry = n_nor == 16
    e = np.where(carry, e + 1, e)
    n_nor = np.where(carry, 8, n_nor)
    code_nor = ((e + 7) << 3) | (n_nor - 8)
    code_nor = np.where(e > 8, CODE_MAX, np.minimum(code_nor, CODE_MAX))

    is_sub = biased < 121  # |a| < 2^-6
    code = np.where(is_sub, n_sub, code_nor)
    code = np.where(biased == 0xFF, np.where(frac != 0, CODE_NAN, CODE_MAX), code)
    return (code | (sign << 7)).astype(np.uint8)


# ---------------------------------------------------------------- BF16 ----

def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) -> float32, exact (BF16 is the top half)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits_rne(x):
    """float32 -> BF16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)
