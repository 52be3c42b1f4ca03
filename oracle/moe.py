"""The steps on either side of the grouped expert GEMMs -- oracle, test
infrastructure.

* Dispatch gather (jp-study.kr doc 258368 ¶1): the activation is quantized
  once, before the MoE dispatch, and the FP8 codes plus their 1x128 scales
  are what is sent to the experts.  On one device that is a row gather of
  (codes, scales) into the expert-sorted order the grouped GEMM reads.
* SwiGLU (tmdrlife.com wr_id=13334 ¶3-¶4): the MoE's SwiGLU operator sits
  between the up- and the down-projection; its inputs are cached in FP8
  with power-of-two scales and its output is recomputed in the backward
  pass.  The down-projection's FP8 input is the 1x128 quantization of the
  SwiGLU output.

Readings taken where the pages are silent:

* SwiGLU(g, u) = silu(g) * u with silu(g) = g / (1 + e^-g); the up-projection
  output holds the gate in its first half of columns and the up values in
  its second half (the weight of the dense up-projection workload stacks
  gate then up).
* The quantized value is the BF16 rounding (nearest, ties to even) of the
  exact SwiGLU value: the tensor an unfused SwiGLU would store in BF16 for
  the quantizer to read.  The GPU forms the value in float32 (hardware exp2
  and reciprocal, one ulp each) in one of two ways, whose relative errors
  are both below ``swiglu_rel_error_bound()`` (about 2^-20.5); where the exact value lies
  within BAND_REL = 2^-19 (relative) of the midpoint between two BF16 numbers
  either neighbour is accepted (``swiglu_accept``); everything else is
  compared bit for bit.
* A gather index outside the source rows gives a zero row and a zero scale.

Pins: tests/test_oracle_moe.py (hand-worked gather, gather commutes with the
1x128 quantizer, closed forms of silu, BF16 rounding against the float32
path and hand-worked ties, SwiGLU with u = 1 and a large gate reducing to
the plain quantizer, the acceptance rule rejecting a planted error, the
error bound composed above against a float32 emulation of the kernel's
arithmetic with its transcendental steps pushed one ulp either way).
"""

import numpy as np

from .e4m3 import bf16_bits_to_f32, encode
from .quantize import FREE, TILE, _tile_scale, quantize_rows

BAND_REL = 2.0 ** -19   # ambiguity band around a BF16 rounding midpoint
BAND_ABS = 2.0 ** -140  # float32 subnormal results carry absolute errors


def swiglu_rel_error_bound(exp2_ulp=1.0, rcp_ulp=1.0):
    """Bound on |y32 - y| / |y| for both float32 forms of the SwiGLU the GPU
    takes (the larger of the two bounds below); the band BAND_REL must
    contain it."""
    return max(swiglu_rel_error_bound_general(exp2_ulp, rcp_ulp),
               swiglu_rel_error_bound_direct(exp2_ulp, rcp_ulp))


def swiglu_rel_error_bound_direct(exp2_ulp=1.0, rcp_ulp=1.0, gate_min=-64.0):
    """First-order bound on |y32 - y| / |y| for the form the GPU takes when
    every gate of a chunk is at least ``gate_min`` (u = 2^-24):

    * e^-g = 2^(-g c1) e^(-g k), c1 = 47274 / 2^15 (log2(e) to 16
      significant bits, so g c1 is exact for a BF16 g) and
      k = 1 - c1 ln 2 = 4.8885e-6 carried as RN32(k): the hardware exp2 of
      the exact argument (exp2_ulp ulp, relative 2u * exp2_ulp) times
      1 - g k by one fused multiply-add (one rounding, u), dropping the
      second-order term (g k)^2 / 2 (relative, at most 0.83u for
      |g| <= 64); g * RN32(k) is off by at most 2u relative, which moves
      1 - g k by less than 2u * 3.2e-4:
      e_e = 2u * exp2_ulp + u + (g_max k)^2 / 2 + 2u * g_max k;
    * 1 + e^-g rounds (u) and carries e's error scaled by e / (1 + e) <= 1,
      the hardware reciprocal adds rcp_ulp ulp (2u * rcp_ulp):
      e_r = u + e_e + 2u * rcp_ulp;
    * g * r and (g * r) * up: two more roundings, 2u.
    """
    u = 2.0 ** -24
    gk = abs(gate_min) * 4.888495152143634e-6
    e_e = 2 * u * exp2_ulp + u + gk * gk / 2 + 2 * u * gk
    e_r = u + e_e + 2 * u * rcp_ulp
    return e_r + 2 * u


def swiglu_rel_error_bound_general(exp2_ulp=1.0, rcp_ulp=1.0):
    """First-order bound on |y32 - y| / |y| for the form the GPU takes for
    any gate (chunks with a gate below -64), composed from the error of
    each step (u = 2^-24, the float32 unit roundoff):

    * exponent reduction x log2(e) = n + f with log2(e) carried as
      RN32(log2 e) + RN32(remainder) and two fused multiply-adds: |df| <= 2u
      (two roundings of a result below 1/2 in magnitude; the 48-bit
      log2(e) and |x| <= 104 add below 2^-41), so 2^f is off by a factor
      2^df, relative ln(2) * 2u;
    * the hardware exp2 on f: exp2_ulp ulp, relative 2u * exp2_ulp; the exact
      ldexp adds nothing (subnormal t is covered by BAND_ABS):
      e_t = ln(2) * 2u + 2u * exp2_ulp;
    * 1 + t rounds (u) and carries t's error scaled by t / (1 + t) <= 1/2;
      the hardware reciprocal: rcp_ulp ulp (2u * rcp_ulp):
      e_r = u + e_t / 2 + 2u * rcp_ulp;
    * sigma = t * r for g < 0 (the larger case): e_t + e_r + u;
    * g * sigma and (g * sigma) * up: two more roundings, 2u.

    The band BAND_REL must contain this bound; the margin covers the
    hardware transcendentals' documented one-ulp accuracy being exceeded by
    up to a factor of about three.
    """
    u = 2.0 ** -24
    e_t = np.log(2.0) * 2 * u + 2 * u * exp2_ulp
    e_r = u + e_t / 2 + 2 * u * rcp_ulp
    return e_t + e_r + u + 2 * u


def gather_rows(codes, scales, index):
    """Rows ``index`` of (codes [rows, cols], scales [rows, nb]); an index
    outside [0, rows) gives a zero row and a zero scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32)
    idx = np.asarray(index, dtype=np.int64)
    rows = codes.shape[0]
    out_c = np.zeros((idx.size, codes.shape[1]), dtype=np.uint8)
    out_s = np.zeros((idx.size, scales.shape[1]), dtype=np.float32)
    ok = (idx >= 0) & (idx < rows)
    out_c[ok] = codes[idx[ok]]
    out_s[ok] = scales[idx[ok]]
    return out_c, out_s


def silu(g):
    """g * sigmoid(g) in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_exact(x_bits):
    """silu(gate) * up in float64 for BF16 bits x = [gate | up] ([rows, 2I])."""
    xb = np.asarray(x_bits, dtype=np.uint16)
    inter = xb.shape[1] // 2
    x = bf16_bits_to_f32(xb).astype(np.float64)
    return silu(x[:, :inter]) * x[:, inter:]


def _bf16_grid(v):
    """(lower, upper) neighbouring BF16 values of float64 v (lower <= v <=
    upper; equal when v is a BF16 value) and the quantum between them."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))  # a = m * 2^e, m in [0.5, 1)
    # 8 significant bits for normals; the fixed quantum 2^-133 below 2^-126
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    lo = np.floor(v / q) * q
    hi = lo + np.where(lo == v, 0.0, q)
    return lo, hi, q


def round_bf16(v):
    """float64 -> nearest BF16 value (ties to even), as float64."""
    v = np.asarray(v, dtype=np.float64)
    lo, hi, q = _bf16_grid(v)
    mid = lo + q / 2
    even_lo = np.mod(np.round(lo / q), 2) == 0
    r = np.where(v < mid, lo, np.where(v > mid, hi, np.where(even_lo, lo, hi)))
    return np.where(r == 0, np.copysign(0.0, v), r)  # a zero result keeps the sign of v


def bf16_bits(v):
    """BF16 bit patterns of float64 values that are BF16 values (sign of
    zero kept)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def swiglu_bf16_bits(x_bits):
    """The BF16 SwiGLU output (bits [rows, I]) of BF16 bits x = [gate | up]."""
    return bf16_bits(round_bf16(swiglu_exact(x_bits)))


def swiglu_quantize(x_bits, mode=FREE):
    """1x128 quantization of the BF16 SwiGLU output: (codes [rows, I],
    scales [rows, ceil(I/128)])."""
    return quantize_rows(swiglu_bf16_bits(x_bits), mode)


def swiglu_candidates(x_bits):
    """BF16 values (float64) the GPU may produce for each output: (first,
    second); second equals first where the exact value is not within the
    ambiguity band of a rounding midpoint."""
    y = swiglu_exact(x_bits)
    r = round_bf16(y)
    lo, hi, q = _bf16_grid(y)
    mid = lo + q / 2
    near = (lo != hi) & (np.abs(y - mid) <= BAND_REL * np.abs(y) + BAND_ABS)
    other = np.where(r == lo, hi, lo)
    other = np.where(other == 0, np.copysign(0.0, y), other)
    return r, np.where(near, other, r)


def swiglu_accept(x_bits, mode, codes_gpu, scales_gpu):
    """Boolean [rows, nb]: tile (r, b) of the GPU output is the 1x128
    quantization of some choice of acceptable BF16 SwiGLU values.

    The scale must be the scale of a possible max-abs and each code the code
    of one of its element's candidates under that scale.  The possible
    max-abs values are the largest of the smaller candidates and the largest
    of the larger ones: when they differ they belong to one element and are
    adjacent BF16 numbers, so nothing lies between them.
    """
    c1, c2 = swiglu_candidates(x_bits)
    rows, inter = c1.shape
    nb = -(-inter // TILE)
    got_c = np.asarray(codes_gpu, dtype=np.uint8)[:, :inter]
    got_s = np.asarray(scales_gpu, dtype=np.float32)
    ok = np.zeros((rows, nb), dtype=bool)
    for b in range(nb):
        sl = slice(b * TILE, min(inter, (b + 1) * TILE))
        a1, a2 = np.abs(c1[:, sl]), np.abs(c2[:, sl])
        low = np.max(np.minimum(a1, a2), axis=1).astype(np.float32)
        high = np.max(np.maximum(a1, a2), axis=1).astype(np.float32)
        s = got_s[:, b]
        s_ok = (_tile_scale(low, mode) == s) | (_tile_scale(high, mode) == s)
        e1 = _codes_under(c1[:, sl], s[:, None])
        e2 = _codes_under(c2[:, sl], s[:, None])
        got = got_c[:, sl]
        ok[:, b] = s_ok & np.all((got == e1) | (got == e2), axis=1)
    return ok


def _codes_under(v, s):
    """E4M3 codes of BF16 values v (float64) with tile scales s ([rows, 1]
    float32), as the 1x128 quantizer forms them: RN32(v / s), or v itself
    for a zero scale."""
    vf = v.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = vf / s
    q = np.where(s == 0, vf, q)
    return encode(q.astype(np.float32))
