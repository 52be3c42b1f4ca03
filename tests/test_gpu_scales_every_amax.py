"""Every quantizer kernel's tile scale for every positive finite BF16 max-abs
(GPU), against the oracle.

jp-study.kr doc 258368 ¶1 fixes the scale of a 1x128 tile or a 128x128
block by its max-abs (tmdrlife.com wr_id=13334 ¶4 for the power-of-two
mode).  The kernels form the free scale RN32(amax / 448) and the reciprocal
they divide by without an IEEE division; here each of the 32,639 positive
finite BF16 values is the max-abs of one tile (the other 127 elements of
the tile are smaller, random signs), and every kernel that quantizes tiles
must return the oracle's scale bit for bit, in both scale modes:

* the 1x128 row quantizer (codes compared in full too);
* the 128x1 token-axis quantizer on the transpose (codes in full);
* the 128x128 block quantizer, each block holding one such tile in its
  first row and zeros elsewhere (first-row codes against the oracle's row
  codes, every other code the E4M3 zero);
* the dual-orientation block quantizer (both scale arrays) and the combined
  activation + weight launch (identical to the separate calls).
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
from oracle import quantize as Q
from oracle.e4m3 import bf16_bits_to_f32
from tests.gpu_util import assert_codes_equal, assert_scales_equal, dev_bf16, host, host_codes, need_gpu, say

pytestmark = pytest.mark.gpu

AMAX = np.arange(1, 0x7F80, dtype=np.uint16)  # every positive finite BF16 pattern


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _tiles():
    """[32639, 128] BF16 bits: row i has max-abs AMAX[i] at column 37i mod 128."""
    rng = np.random.default_rng(5)
    n = AMAX.size
    # positive BF16 patterns order like their values, so a pattern below
    # AMAX[i] is a magnitude below it
    t = (rng.random((n, 128)) * AMAX[:, None]).astype(np.uint16)
    t |= (rng.random((n, 128)) < 0.5).astype(np.uint16) << 15
    idx = np.arange(n)
    t[idx, (idx * 37) % 128] = AMAX | ((idx & 1).astype(np.uint16) << 15)
    return t


def _want_scales(mode):
    return Q._tile_scale(bf16_bits_to_f32(AMAX), mode).astype(np.float32)


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_row_and_token_axis_scales_every_amax(mode):
    t = _tiles()
    want = _want_scales(mode)
    say(f"[scales] row quantizer, every BF16 amax, {mode}")
    c, s = fp8q.quantize_act(dev_bf16(t), tile_axis="row", scale_mode=mode)
    assert_scales_equal(host(s)[:, 0], want, f"row scales {mode}")
    wc, ws = Q.quantize_rows(t, mode)
    assert_scales_equal(ws[:, 0], want, "oracle row scales (self-check)")
    assert_codes_equal(host_codes(c), wc, f"row codes {mode}")
    say(f"[scales] token-axis quantizer, every BF16 amax, {mode}")
    tt = np.ascontiguousarray(t.T)  # [128 tokens, 32639 features]
    c, s = fp8q.quantize_act(dev_bf16(tt), tile_axis="token_t", scale_mode=mode)
    assert_scales_equal(host(s)[:, 0], want, f"token-axis scales {mode}")
    assert_codes_equal(host_codes(c), wc, f"token-axis codes {mode}")


@pytest.mark.parametrize("mode", ["free", "pow2"])
def test_block_scales_every_amax(mode):
    t = _tiles()
    n = AMAX.size
    want = _want_scales(mode)
    # W [128, 128 n]: block j holds tile j in its first row, zeros below
    w = np.zeros((128, 128 * n), dtype=np.uint16)
    w[0] = t.reshape(-1)
    wd = dev_bf16(w)
    del w
    wc_row, _ = Q.quantize_rows(t, mode)
    say(f"[scales] block quantizer, every BF16 amax, {mode}")
    c, s = fp8q.quantize_weight(wd, scale_mode=mode)
    assert_scales_equal(host(s)[0], want, f"block scales {mode}")
    assert_codes_equal(host_codes(c[0:1]).reshape(n, 128), wc_row, f"block first-row codes {mode}")
    assert int(torch.count_nonzero(c[1:])) == 0, "codes of the zero rows must be the E4M3 zero"
    say(f"[scales] dual-orientation block quantizer, every BF16 amax, {mode}")
    c2, s2, ct, st = fp8q.quantize_weight_t(wd, scale_mode=mode)
    assert torch.equal(c2, c) and torch.equal(s2.view(torch.int32), s.view(torch.int32))
    assert_scales_equal(host(st)[:, 0], want, f"transposed block scales {mode}")
    assert torch.equal(ct.t().contiguous(), c), "transposed codes are the transpose of the codes"
    del c2, s2, ct, st
    say(f"[scales] activation + weight in one launch, every BF16 amax, {mode}")
    # the combined launch needs the activation's K to equal the weight's K:
    # activation rows of 128 * n columns, the tiles laid end to end
    a = dev_bf16(np.tile(t.reshape(1, -1), (2, 1)))
    ac, asc, lc, lsc = fp8q.quantize_linear(a, wd, act_scale_mode=mode, weight_scale_mode=mode)
    ac0, as0 = fp8q.quantize_act(a, tile_axis="row", scale_mode=mode)
    assert torch.equal(ac, ac0) and torch.equal(asc.view(torch.int32), as0.view(torch.int32))
    assert torch.equal(lc, c) and torch.equal(lsc.view(torch.int32), s.view(torch.int32))
    assert_scales_equal(host(asc)[0], want, f"combined launch activation scales {mode}")
