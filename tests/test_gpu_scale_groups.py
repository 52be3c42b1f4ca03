"""GPU parity across the GEMMs' scale staging.

The kernels move the per-row and per-column scales into LDS four K blocks at
a time (one load instruction covers 16 rows x 4 blocks; every K block's
refill brings a quarter of the next group).  These cases put K block counts
that leave a partial last group (k/128 = 6, 7) or run over several groups
(9, 13) through every accumulation form, the grouped GEMM and the weight
gradient, with 1x128 tiles and 128x128 blocks whose magnitudes differ by up
to 2^24 from block to block and row to row, so a scale taken from the wrong
row, block or group moves an output far outside the tolerance.

Acceptance as in the other GEMM parity tests: the FP32-grade forms (and the
power-of-two one, on operands quantized with power-of-two scales) within
1e-5 * S + 1e-6 of the oracle on every element; the FP8-unit forms against
the hardware model of that unit (tests/fp8_unit_model.py, no parity claim)
with the allowances of tests/test_gpu_native.py, on a sample that covers every row and every column
(so every scale entry).
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from oracle import gemm as G, quantize as Q
from tests import fp8_unit_model as unit
from tests.gpu_util import dev, host, need_gpu, say
from tests.test_gpu_gemm import _accept
from tests.test_gpu_native import _accept_chained, _accept_model

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _sample(rng, m, n):
    """Output elements covering every row and every column: all rows at the
    columns around each 128-column edge, all columns at the rows around each
    16-, 64- and 128-row edge, and 3000 more at random."""
    cs = sorted({c for c in (0, 1, 127, 128, 129, 255, 256, n - 1) if 0 <= c < n})
    rs = sorted({r for r in (0, 15, 16, 63, 64, 127, 128, m - 1) if 0 <= r < m})
    rows = np.concatenate([np.repeat(np.arange(m), len(cs)), np.repeat(rs, n), rng.integers(0, m, 3000)])
    cols = np.concatenate([np.tile(cs, m), np.tile(np.arange(n), len(rs)), rng.integers(0, n, 3000)])
    return rows, cols


def _tile_spread(rng, rows, k):
    """BF16 [rows, k] whose 1x128 tiles carry independent factors 2^-12..2^12."""
    e = rng.integers(-12, 13, (rows, k // 128))
    x = rng.standard_normal((rows, k)) * np.exp2(np.repeat(e, 128, axis=1))
    return synth.bf16_rne(x.astype(np.float32))


def _block_spread(rng, n, k):
    """BF16 [n, k] ~N(0, 0.02) whose 128x128 blocks carry factors 2^-12..2^12."""
    e = rng.integers(-12, 13, ((n + 127) // 128, k // 128))
    f = np.exp2(np.repeat(np.repeat(e, 128, axis=0)[:n], 128, axis=1))
    return synth.bf16_rne((rng.standard_normal((n, k)) * 0.02 * f).astype(np.float32))


@pytest.mark.parametrize("nkb", [6, 7, 9, 13])
@pytest.mark.parametrize("acc", ["fp32", "fp8_mfma", "fp8_mfma_scaled", "fp32_pow2"])
def test_dense_scale_groups(nkb, acc):
    m, n, k = 200, 260, 128 * nkb
    rng = np.random.default_rng(100 + nkb)
    mode = Q.POW2 if acc in ("fp8_mfma_scaled", "fp32_pow2") else Q.FREE
    a_c, a_s = Q.quantize_rows(_tile_spread(rng, m, k), mode)
    w_c, w_s = Q.quantize_blocks(_block_spread(rng, n, k), mode)
    say(f"[scale groups] dense {m}x{n}x{k} acc={acc}")
    c = fp8q.gemm(dev(a_c), dev(a_s), dev(w_c), dev(w_s), out_dtype=torch.float32, acc=acc)
    if acc in ("fp32", "fp32_pow2"):
        ref, s = G.gemm(a_c, a_s, w_c, w_s)
        _accept(c, ref, s, f"dense k/128={nkb}")
        return
    rows, cols = _sample(rng, m, n)
    got = c[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()]
    if acc == "fp8_mfma":
        ref, s, t = unit.gemm_at_mfma(a_c, a_s, w_c, w_s, rows, cols)
        _accept_model(got, ref, s, t, f"dense fp8 unit k/128={nkb}")
    else:
        _accept_chained(host(got).astype(np.float64), a_c, a_s, w_c, w_s, rows, cols,
                        f"dense scaled k/128={nkb}")


@pytest.mark.parametrize("n", [256, 328])
@pytest.mark.parametrize("acc", ["fp32", "fp8_mfma", "fp32_pow2"])
def test_grouped_scale_groups(acc, n):
    # four experts of 0, 70, 300 and 129 rows (tiles of every wave layout),
    # N a multiple of the tile width or not (a last N tile of 72 columns,
    # with a partial W block)
    counts = np.array([0, 70, 300, 129])
    offs = np.zeros(len(counts) + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    rows, k = int(offs[-1]), 128 * 7
    rng = np.random.default_rng(7 + n)
    mode = Q.POW2 if acc == "fp32_pow2" else Q.FREE
    a_c, a_s = Q.quantize_rows(_tile_spread(rng, rows, k), mode)
    q = [Q.quantize_blocks(_block_spread(rng, n, k), mode) for _ in counts]
    wc, ws = np.stack([c for c, _ in q]), np.stack([s for _, s in q])
    say(f"[scale groups] grouped {counts.tolist()} N={n} K={k} acc={acc}")
    c = fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws), out_dtype=torch.float32, acc=acc)
    if acc in ("fp32", "fp32_pow2"):
        ref, s = G.grouped_gemm(a_c, a_s, offs, wc, ws)
        _accept(c, ref, s, f"grouped k/128=7 N={n}")
        return
    for gi in range(len(counts)):
        lo, hi = int(offs[gi]), int(offs[gi + 1])
        if hi == lo:
            continue
        rr, cc = _sample(rng, hi - lo, n)
        got = c[torch.from_numpy(rr + lo).cuda(), torch.from_numpy(cc).cuda()]
        ref, s, t = unit.gemm_at_mfma(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi], rr, cc)
        _accept_model(got, ref, s, t, f"grouped fp8 unit N={n} expert {gi}")


@pytest.mark.parametrize("nkb", [7, 9])
@pytest.mark.parametrize("acc", ["fp32", "fp8_mfma", "fp32_pow2"])
def test_wgrad_scale_groups(nkb, acc):
    t_tok, nout, kin = 128 * nkb, 200, 300
    rng = np.random.default_rng(200 + nkb)
    # token-axis tiles: factors vary per 128-token block and per column
    e_dy = np.repeat(rng.integers(-12, 13, (nkb, nout)), 128, axis=0)
    e_x = np.repeat(rng.integers(-12, 13, (nkb, kin)), 128, axis=0)
    dy = synth.bf16_rne((rng.standard_normal((t_tok, nout)) * np.exp2(e_dy)).astype(np.float32))
    x = synth.bf16_rne((rng.standard_normal((t_tok, kin)) * np.exp2(e_x)).astype(np.float32))
    mode = Q.POW2 if acc == "fp32_pow2" else Q.FREE
    dy_c, dy_s = Q.quantize_token_t(dy, mode)
    x_c, x_s = Q.quantize_token_t(x, mode)
    say(f"[scale groups] wgrad T={t_tok} {nout}x{kin} acc={acc}")
    dw = fp8q.wgrad(dev(dy_c), dev(dy_s), dev(x_c), dev(x_s), acc=acc)
    if acc in ("fp32", "fp32_pow2"):
        ref, s = G.wgrad(dy_c, dy_s, x_c, x_s)
        _accept(dw, ref, s, f"wgrad k/128={nkb}")
        return
    rr, cc = _sample(rng, nout, kin)
    got = dw[torch.from_numpy(rr).cuda(), torch.from_numpy(cc).cuda()]
    ref, s, t = unit.gemm_at_mfma(dy_c, dy_s, x_c, x_s, rr, cc, w_block_rows=False)
    _accept_model(got, ref, s, t, f"wgrad fp8 unit k/128={nkb}")
