"""Block-scaled FP8 GEMMs and the output acceptance rule -- oracle.

tmdrlife.com wr_id=13334 ¶3 and gnrental.net wr_id=40936 ¶4: once the
accumulation interval is reached, the partial products are moved to FP32
registers, multiplied by the scaling factors and added there.
jp-study.kr doc 258368 ¶3: that interval is 128 elements of K.  Since each
128-element K interval is one activation tile and one weight block, the
result the method reaches (up to rounding order) has the plain definition

    C[m, n] = sum_b  sa[m, b] * sw[n // 128, b] * sum_{k in block b} qa[m, k] * qw[n, k]

with qa, qw the decoded E4M3 values.  That definition is written out here.
Every E4M3 value is an integer multiple of 2^-9 with magnitude below 2^18 *
2^-9, so each block's partial sum is an integer multiple of 2^-18 below 2^25
in magnitude: it is exact in float64 whatever the summation order.  The scale
product of two float32 values is exact in float64 (48 significant bits).
Only the outer sum over blocks rounds, by at most about n_blocks * 2^-53
relative to S below.

S[m, n] = sum_b |sa * sw| * sum_k |qa| * |qw| is the sum of |a_i * b_i| over
the dequantized operands; the acceptance rule for a GPU result c is

    FP32 output:  |c - C| <= 1e-5 * S + 1e-6
    BF16 output:  c is the round-to-nearest-even BF16 of some float32 value
                  in [C - tol, C + tol], tol = 1e-5 * S + 1e-6  (an interval
                  test, since rounding is monotone)
    E4M3 output (the BF16 output quantized per 1x128 tile along N, the
                  producer-side answer to tmdrlife.com wr_id=13334 ¶1): each
                  tile is the quantization of some BF16 tensor that passes
                  the BF16 rule (``accept_quantized``)

jp-study.kr doc 258368 ¶3 (Wgrad in FP8): the weight gradient is the same
contraction over the token axis with both operands scaled per 128 tokens and
per row, dW[n, c] = sum_b sdy[n, b] * sx[c, b] * sum_{t in b} qdy[n, t] qx[c, t].

Pins: tests/test_oracle_gemm.py (exact integer + Fraction brute force on the
tiny-linear shape, constant-operand closed form, selector weights, zero
scales, grouped == per-group dense, Wgrad == dense when scales are constant
per block, the BF16 interval rule on hand-made cases, the quantized-output
rule accepting the quantization of the exact result and rejecting planted
code and scale errors, accepting any quantization inside a wide zero-result
band, and its attained-scale test against all 32,640 enumerated BF16
scales).
"""

import numpy as np

from .e4m3 import decode_int

TILE = 128
TWO_M18 = 2.0 ** -18


def _block_partials_int(a_codes, w_codes, b):
    """Exact per-block partial sums in units of 2^-18, as float64 (exact)."""
    sl = slice(b * TILE, (b + 1) * TILE)
    ia = decode_int(a_codes[:, sl]).astype(np.float64)
    iw = decode_int(w_codes[:, sl]).astype(np.float64)
    return ia @ iw.T, np.abs(ia) @ np.abs(iw).T


def gemm(a_codes, a_scales, w_codes, w_scales):
    """Dense C = A . W^T with 1x128 activation scales and 128x128 weight scales.

    a_codes [M, K], a_scales [M, K/128], w_codes [N, K],
    w_scales [ceil(N/128), K/128].  Returns (C, S) as float64 [M, N].
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    w_codes = np.asarray(w_codes, dtype=np.uint8)
    m, k = a_codes.shape
    n = w_codes.shape[0]
    if k % TILE:
        raise ValueError("K must be a multiple of 128")
    nb = k // TILE
    sa = np.asarray(a_scales, dtype=np.float32).astype(np.float64)
    sw = np.repeat(np.asarray(w_scales, dtype=np.float32).astype(np.float64), TILE, axis=0)[:n]
    c = np.zeros((m, n))
    s = np.zeros((m, n))
    for b in range(nb):
        p, pabs = _block_partials_int(a_codes, w_codes, b)
        scale = sa[:, b][:, None] * sw[:, b][None, :]  # exact in float64
        c += scale * (p * TWO_M18)
        s += np.abs(scale) * (pabs * TWO_M18)
    return c, s


def grouped_gemm(a_codes, a_scales, offsets, w_codes, w_scales):
    """Per-group dense GEMM: rows [offsets[g], offsets[g+1]) use W[g].

    a_codes [rows, K]; offsets int [G+1]; w_codes [G, N, K];
    w_scales [G, ceil(N/128), K/128].  Returns (C, S) float64 [rows, N]; rows
    not covered by any group are NaN.
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    offsets = [int(v) for v in offsets]
    g_count = len(offsets) - 1
    n = np.asarray(w_codes).shape[1]
    c = np.full((a_codes.shape[0], n), np.nan)
    s = np.full((a_codes.shape[0], n), np.nan)
    for g in range(g_count):
        lo, hi = offsets[g], offsets[g + 1]
        if hi <= lo:
            continue
        cg, sg = gemm(a_codes[lo:hi], np.asarray(a_scales)[lo:hi], w_codes[g], w_scales[g])
        c[lo:hi] = cg
        s[lo:hi] = sg
    return c, s


def wgrad(dy_t_codes, dy_scales, x_t_codes, x_scales):
    """dW = dY^T X over the token axis, both operands 128x1 token tiles.

    dy_t_codes [Nout, T], dy_scales [Nout, T/128], x_t_codes [Kin, T],
    x_scales [Kin, T/128].  Returns (dW, S) float64 [Nout, Kin].
    """
    dy = np.asarray(dy_t_codes, dtype=np.uint8)
    xt = np.asarray(x_t_codes, dtype=np.uint8)
    nout, t = dy.shape
    kin = xt.shape[0]
    if t % TILE:
        raise ValueError("T must be a multiple of 128")
    sdy = np.asarray(dy_scales, dtype=np.float32).astype(np.float64)
    sx = np.asarray(x_scales, dtype=np.float32).astype(np.float64)
    c = np.zeros((nout, kin))
    s = np.zeros((nout, kin))
    for b in range(t // TILE):
        p, pabs = _block_partials_int(dy, xt, b)
        scale = sdy[:, b][:, None] * sx[:, b][None, :]
        c += scale * (p * TWO_M18)
        s += np.abs(scale) * (pabs * TWO_M18)
    return c, s


def gemm_at(a_codes, a_scales, w_codes, w_scales, rows, cols, w_block_rows=True):
    """C and S at sampled positions (rows[i], cols[i]) only, one by one.

    Same definition as ``gemm`` (w_block_rows=True: weight scales per 128-row
    block) or ``wgrad`` (w_block_rows=False: weight scales per row), evaluated
    for a list of output elements so full-size problems can be checked.
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    w_codes = np.asarray(w_codes, dtype=np.uint8)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    k = a_codes.shape[1]
    nb = k // TILE
    ia = decode_int(a_codes[rows]).astype(np.float64).reshape(-1, nb, TILE)
    iw = decode_int(w_codes[cols]).astype(np.float64).reshape(-1, nb, TILE)
    p = np.einsum("ibk,ibk->ib", ia, iw) * TWO_M18  # exact per block
    pabs = np.einsum("ibk,ibk->ib", np.abs(ia), np.abs(iw)) * TWO_M18
    sa = np.asarray(a_scales, dtype=np.float32).astype(np.float64)[rows]
    wr = cols // TILE if w_block_rows else cols
    sw = np.asarray(w_scales, dtype=np.float32).astype(np.float64)[wr]
    scale = sa * sw
    return (scale * p).sum(axis=1), (np.abs(scale) * pabs).sum(axis=1)


# ----------------------------------------------------- acceptance rule ----

def tolerance(s):
    return 1e-5 * np.asarray(s, dtype=np.float64) + 1e-6


def accept_f32(c_gpu, c_ref, s_ref):
    """Elementwise |c_gpu - C| <= 1e-5 * S + 1e-6 (boolean array)."""
    err = np.abs(np.asarray(c_gpu, dtype=np.float64) - c_ref)
    return err <= tolerance(s_ref)


def _f32_toward(x, up):
    """Nearest float32 >= x (up=True) or <= x (up=False), for float64 x."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    f64 = f.astype(np.float64)
    if up:
        return np.where(f64 < x, np.nextafter(f, np.float32(np.inf)), f)
    return np.where(f64 > x, np.nextafter(f, np.float32(-np.inf)), f)


def _bf16_rne_value(f32):
    """RNE rounding of float32 values to BF16, returned as float64 values."""
    u = np.ascontiguousarray(np.asarray(f32, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def accept_bf16(c_gpu_bf16_bits, c_ref, s_ref):
    """BF16 output rule: c_gpu in [RNE(lo32), RNE(hi32)] (boolean array).

    lo32 / hi32 are the float32 values closest to C -/+ tol from inside the
    interval, so the accepted set is exactly the BF16 roundings of float32
    values within tolerance.
    """
    tol = tolerance(s_ref)
    lo = _bf16_rne_value(_f32_toward(c_ref - tol, up=True))
    hi = _bf16_rne_value(_f32_toward(c_ref + tol, up=False))
    v = (np.asarray(c_gpu_bf16_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    v = v.astype(np.float64)
    return (v >= lo) & (v <= hi)


def _scale_attained(s, mode):
    """True where the float32 scale s (>= 0) is the tile scale of some BF16
    value v >= 0, i.e. lies in the image of v -> scale(v).

    Power-of-two scales: s is 0 or a power of two between the scales of the
    smallest and the largest positive BF16 values.  Free scales
    s = RN32(v / 448): v then lies within 448 * ulp(s) / 2 of 448 * s, an
    interval that holds at most one BF16 value, one of the BF16 neighbours
    of 448 * s; those are tried.
    """
    from .quantize import FREE, _tile_scale

    s = np.asarray(s, dtype=np.float32)
    if mode != FREE:
        ends = _tile_scale((np.array([1, 0x7F7F], dtype=np.uint32) << 16).view(np.float32), mode)
        m, _ = np.frexp(s.astype(np.float64))
        return (s == 0) | ((m == 0.5) & (s >= ends[0]) & (s <= ends[1]))
    with np.errstate(over="ignore"):  # 448 * s beyond float32: no BF16 value reaches it
        v = (s.astype(np.float64) * 448.0).astype(np.float32)
    b = (np.ascontiguousarray(v).view(np.uint32) >> 16).astype(np.int64)
    hit = s == 0
    for d in (-1, 0, 1):
        cand = (np.clip(b + d, 0, 0x7F7F).astype(np.uint32) << 16).view(np.float32)
        hit |= _tile_scale(cand, mode) == s
    return hit


def accept_quantized(codes_gpu, scales_gpu, c_ref, s_ref, mode):
    """Quantized-output rule, per 1x128 tile along N (boolean [M, nb]): the
    GPU tile must be the 1x128 quantization (oracle.quantize) of some BF16
    tensor that passes ``accept_bf16`` elementwise.

    Each element's admissible BF16 values form an interval [lo, hi]
    (``accept_bf16``), so its admissible magnitudes run from min_mag (0 when
    the interval holds 0) to max_mag.  The tile max-abs of an admissible
    tensor can be any BF16 value between a_lo = max(min_mag) and
    a_hi = max(max_mag) (set the element with the largest max_mag to it and
    every other element to its min_mag).  The scale is a non-decreasing
    function of the max-abs, so the scales of those tensors are exactly the
    attained scales between scale(a_lo) and scale(a_hi); each code must then
    lie between the codes of its interval's ends under the GPU's scale (the
    quotient and the E4M3 rounding are monotone in the value).
    """
    from .e4m3 import decode, encode
    from .quantize import TILE, _tile_scale

    c_ref = np.asarray(c_ref, dtype=np.float64)
    tol = tolerance(s_ref)
    lo = _bf16_rne_value(_f32_toward(c_ref - tol, up=True))
    hi = _bf16_rne_value(_f32_toward(c_ref + tol, up=False))
    min_mag = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    max_mag = np.maximum(np.abs(lo), np.abs(hi))
    m, n = c_ref.shape
    nb = -(-n // TILE)
    codes_gpu = np.asarray(codes_gpu, dtype=np.uint8)[:, :n]
    scales_gpu = np.asarray(scales_gpu, dtype=np.float32)
    ok = np.zeros((m, nb), dtype=bool)
    for b in range(nb):
        sl = slice(b * TILE, min(n, (b + 1) * TILE))
        a_lo = np.max(min_mag[:, sl], axis=1).astype(np.float32)
        a_hi = np.max(max_mag[:, sl], axis=1).astype(np.float32)
        s = scales_gpu[:, b]
        s_ok = (s >= _tile_scale(a_lo, mode)) & (s <= _tile_scale(a_hi, mode)) & _scale_attained(s, mode)

        def codes_of(v):
            vf = v.astype(np.float32)
            with np.errstate(divide="ignore", invalid="ignore"):
                q = vf / s[:, None]
            return decode(encode(np.where(s[:, None] == 0, vf, q).astype(np.float32)))

        d_lo, d_hi = codes_of(lo[:, sl]), codes_of(hi[:, sl])
        got = decode(codes_gpu[:, sl])
        c_ok = np.all((got >= np.minimum(d_lo, d_hi)) & (got <= np.maximum(d_lo, d_hi)), axis=1)
        ok[:, b] = s_ok & c_ok
    return ok
