"""Online max-abs quantizers -- oracle, test infrastructure.

jp-study.kr doc 258368 ¶1: the maximum absolute value is taken online for
every 1x128 activation tile and every 128x128 weight block, and it sets that
tile's scaling factor.  tmdrlife.com wr_id=13334 ¶4 and gnrental.net
wr_id=40936 ¶3: for some activations (inputs of the Linear after attention,
SwiGLU inputs in MoE, the activation gradient before MoE down-projections)
the scaling factors are integral powers of 2.

Readings taken where the pages are silent:

* free scale  s = RN32(amax / 448): the max-abs element lands on the largest
  E4M3 magnitude; the code of x is E4M3_RNE(RN32(x / s)), an IEEE float32
  division followed by the E4M3 rounding (the double rounding is part of the
  definition);
* power-of-two scale s = the smallest 2^e with amax / s <= 448, found from
  the exponent and mantissa of amax exactly; then x / s is exact;
* an all-zero tile has s = 0 and signed-zero codes;
* a ragged last tile takes its max over the valid elements only;
* "1x128" runs along the GEMM reduction axis K; weight blocks are 128 rows of
  N by 128 columns of K; for the weight gradient the reduction axis is the
  token axis, so its tiles are 128 tokens x 1 feature and the codes are
  stored transposed (feature-major, tokens contiguous).

Inputs are BF16 bit patterns (uint16 arrays); outputs are uint8 codes and
float32 scales.  Pins: tests/test_oracle_quantize.py (max element -> 0x7E,
half-ulp dequantization bound, exact powers of two, power-of-two
equivariance, negation symmetry, concatenation and row-gather invariance,
hand-worked tiles in tests/golden/quant_tiles.txt).
"""

import math

import numpy as np

from .e4m3 import MAX_FINITE, bf16_bits_to_f32, encode

TILE = 128
FREE = "free"
POW2 = "pow2"


def _tile_scale(amax, mode):
    """Scale for each tile from its float32 max-abs (array of float32)."""
    amax = np.asarray(amax, dtype=np.float32)
    if mode == FREE:
        with np.errstate(divide="ignore", invalid="ignore"):
            s = amax / np.float32(MAX_FINITE)  # IEEE float32 division, RN
        return np.where(amax == 0, np.float32(0), s).astype(np.float32)
    if mode == POW2:
        out = np.zeros(amax.shape, dtype=np.float32)
        flat_a = amax.reshape(-1)
        flat_o = out.reshape(-1)
        for i, a in enumerate(flat_a.tolist()):
            if a == 0.0:
                continue
            f, k = math.frexp(a)  # a = f * 2^k, f in [0.5, 1)
            m, E = 2.0 * f, k - 1  # a = m * 2^E, m in [1, 2)
            e = E - 8 + (1 if m > 1.75 else 0)  # 448 = 1.75 * 2^8
            flat_o[i] = np.float32(math.ldexp(1.0, e))
        return out
    raise ValueError(f"unknown scale mode {mode!r}")


def _quantize_tiles(xf, mode):
    """Quantize rows of xf (float32 [n_tiles, L], padded with NaN) per row."""
    valid = ~np.isnan(xf)
    amax = np.max(np.where(valid, np.abs(xf), np.float32(0)), axis=1)
    s = _tile_scale(amax, mode)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = xf / s[:, None]  # float32 / float32: IEEE RN division (exact for POW2)
    q = np.where(s[:, None] == 0, xf, q)  # zero tile: codes keep the zeros' signs
    codes = encode(np.where(valid, q, np.float32(0)))
    return codes, s


def quantize_rows(x_bits, mode=FREE):
    """1x128 tiles along the columns of x ([rows, cols] BF16 bits).

    Returns (codes uint8 [rows, cols], scales float32 [rows, ceil(cols/128)]).
    """
    xb = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = xb.shape
    nb = -(-cols // TILE)
    xf = np.full((rows, nb * TILE), np.nan, dtype=np.float32)
    xf[:, :cols] = bf16_bits_to_f32(xb)
    codes, s = _quantize_tiles(xf.reshape(rows * nb, TILE), mode)
    codes = codes.reshape(rows, nb * TILE)[:, :cols]
    return np.ascontiguousarray(codes), s.reshape(rows, nb)


def quantize_token_t(x_bits, mode=FREE):
    """128x1 tiles along the rows (token axis) of x ([T, C] BF16 bits).

    Returns (codes uint8 [C, T] -- transposed, tokens contiguous --,
    scales float32 [C, ceil(T/128)]).  A 128x1 tile of x is a 1x128 tile of
    its transpose, so this is quantize_rows applied to x^T.
    """
    xb = np.asarray(x_bits, dtype=np.uint16)
    return quantize_rows(np.ascontiguousarray(xb.T), mode)


def quantize_blocks(w_bits, mode=FREE):
    """128x128 blocks of w ([N, K] BF16 bits).

    Returns (codes uint8 [N, K], scales float32 [ceil(N/128), ceil(K/128)]).
    """
    wb = np.asarray(w_bits, dtype=np.uint16)
    n, k = wb.shape
    bn, bk = -(-n // TILE), -(-k // TILE)
    wf = np.full((bn * TILE, bk * TILE), np.nan, dtype=np.float32)
    wf[:n, :k] = bf16_bits_to_f32(wb)
    # [bn, 128, bk, 128] -> [bn, bk, 128*128]: one row per block
    blocks = wf.reshape(bn, TILE, bk, TILE).transpose(0, 2, 1, 3).reshape(bn * bk, TILE * TILE)
    codes, s = _quantize_tiles(blocks, mode)
    codes = codes.reshape(bn, bk, TILE, TILE).transpose(0, 2, 1, 3).reshape(bn * TILE, bk * TILE)
    return np.ascontiguousarray(codes[:n, :k]), s.reshape(bn, bk)


def dequantize_rows(codes, scales):
    """Dequantized values code * scale (float64) for 1x128 row tiles."""
    from .e4m3 import decode
    c = np.asarray(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), TILE, axis=1)[:, : c.shape[1]]
    return decode(c) * s


def dequantize_blocks(codes, scales):
    """Dequantized values code * scale (float64) for 128x128 blocks."""
    from .e4m3 import decode
    c = np.asarray(codes)
    s = np.repeat(np.repeat(np.asarray(scales, dtype=np.float64), TILE, axis=0), TILE, axis=1)
    return decode(c) * s[: c.shape[0], : c.shape[1]]
