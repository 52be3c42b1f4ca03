"""A seeded sweep of random shapes through the whole path (GPU + oracle).

Each case draws its shapes, scale modes, accumulation form, output dtype
and a padded input row stride from a fixed seed, quantizes on the GPU,
checks codes and scales bit for bit against the oracle, then runs the GEMM
and checks every output element against the oracle at the stated
tolerance |gpu - oracle| <= 1e-5 * S + 1e-6 (BF16 output: the interval
rule).  Inputs have per-row magnitudes spread over 2^-6 .. 2^6 so tile
scales differ widely.  The forms swept are the ones with a float32-grade
parity claim: the default (free or power-of-two scales) and the
power-of-two float32-grade form (power-of-two scales).

* dense: M, N in [1, 700], K = 128 * [1, 12];
* grouped: 1-6 experts of 0-300 rows each (zero included), rows_cap past
  the last offset, N in [1, 600], K = 128 * [1, 8];
* Wgrad: T = 128 * [1, 8] tokens, Nout, Kin in [1, 600], token-axis tiles.
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
import synth
from oracle import gemm as G, quantize as Q
from tests.gpu_util import (assert_codes_equal, assert_scales_equal, dev, dev_bf16, host, host_bf16_bits,
                            host_codes, need_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _bits(rng, rows, cols, std=1.0):
    x = rng.standard_normal((rows, cols)) * std * np.exp2(rng.integers(-6, 7, (rows, 1)))
    return synth.bf16_rne(x.astype(np.float32))


def _padded(bits, rng):
    """BF16 on the GPU with a row stride of cols + 8 * [0, 3] elements."""
    rows, cols = bits.shape
    pad = 8 * int(rng.integers(0, 4))
    full = np.zeros((rows, cols + pad), np.uint16)
    full[:, :cols] = bits
    return dev_bf16(full)[:, :cols]


def _accept(got, ref, s, bf16, what):
    ok = G.accept_bf16(got, ref, s) if bf16 else G.accept_f32(got, ref, s)
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outside the tolerance"


def _out(c):
    if c.dtype == torch.bfloat16:
        return host_bf16_bits(c), True
    return host(c).astype(np.float64), False


@pytest.mark.parametrize("seed", range(12))
def test_dense(seed):
    rng = np.random.default_rng(1000 + seed)
    m, n = (int(v) for v in rng.integers(1, 701, 2))
    k = 128 * int(rng.integers(1, 13))
    acc = ("fp32", "fp32_pow2")[int(rng.integers(0, 2))]
    a_mode = "pow2" if acc == "fp32_pow2" else ("free", "pow2")[int(rng.integers(0, 2))]
    w_mode = "pow2" if acc == "fp32_pow2" else ("free", "pow2")[int(rng.integers(0, 2))]
    out_dtype = (torch.float32, torch.bfloat16)[int(rng.integers(0, 2))]
    a_bits, w_bits = _bits(rng, m, k), _bits(rng, n, k, 0.02)
    say(f"[sweep] dense {m}x{n}x{k} acc={acc} scales={a_mode}/{w_mode} out={out_dtype}")
    a_c, a_s = fp8q.quantize_act(_padded(a_bits, rng), scale_mode=a_mode)
    w_c, w_s = fp8q.quantize_weight(_padded(w_bits, rng), scale_mode=w_mode)
    oa_c, oa_s = Q.quantize_rows(a_bits, Q.POW2 if a_mode == "pow2" else Q.FREE)
    ow_c, ow_s = Q.quantize_blocks(w_bits, Q.POW2 if w_mode == "pow2" else Q.FREE)
    assert_codes_equal(host_codes(a_c), oa_c, "A codes")
    assert_scales_equal(host(a_s), oa_s, "A scales")
    assert_codes_equal(host_codes(w_c), ow_c, "W codes")
    assert_scales_equal(host(w_s), ow_s, "W scales")
    c = fp8q.gemm(a_c.contiguous(), a_s, w_c.contiguous(), w_s, out_dtype=out_dtype, acc=acc)
    ref, s = G.gemm(oa_c, oa_s, ow_c, ow_s)
    got, bf16 = _out(c)
    _accept(got, ref, s, bf16, f"dense {m}x{n}x{k} {acc}")


@pytest.mark.parametrize("seed", range(8))
def test_grouped(seed):
    rng = np.random.default_rng(2000 + seed)
    g = int(rng.integers(1, 7))
    counts = rng.integers(0, 301, g)
    counts[int(rng.integers(0, g))] = 0 if g > 1 else counts[0]   # an empty expert when there are several
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows_cap = int(offs[-1]) + int(rng.integers(0, 40))
    n = int(rng.integers(1, 601))
    k = 128 * int(rng.integers(1, 9))
    acc = ("fp32", "fp32_pow2")[int(rng.integers(0, 2))]
    mode = Q.POW2 if acc == "fp32_pow2" else (Q.FREE, Q.POW2)[int(rng.integers(0, 2))]
    out_dtype = (torch.float32, torch.bfloat16)[int(rng.integers(0, 2))]
    say(f"[sweep] grouped experts {counts.tolist()} cap {rows_cap} n {n} k {k} acc={acc}")
    a_c, a_s = Q.quantize_rows(_bits(rng, max(rows_cap, 1), k), mode)
    a_c, a_s = a_c[:rows_cap], a_s[:rows_cap]
    wq = [Q.quantize_blocks(_bits(rng, n, k, 0.02), mode) for _ in range(g)]
    wc, ws = np.stack([c for c, _ in wq]), np.stack([s for _, s in wq])
    c = fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws), out_dtype=out_dtype, acc=acc)
    got, bf16 = _out(c)
    for gi in range(g):
        lo, hi = int(offs[gi]), int(offs[gi + 1])
        if hi == lo:
            continue
        ref, s = G.gemm(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi])
        _accept(got[lo:hi], ref, s, bf16, f"expert {gi} ({hi - lo} rows)")


@pytest.mark.parametrize("seed", range(8))
def test_wgrad(seed):
    rng = np.random.default_rng(3000 + seed)
    t = 128 * int(rng.integers(1, 9))
    nout, kin = (int(v) for v in rng.integers(1, 601, 2))
    acc = ("fp32", "fp32_pow2")[int(rng.integers(0, 2))]
    mode = "pow2" if acc == "fp32_pow2" else ("free", "pow2")[int(rng.integers(0, 2))]
    qm = Q.POW2 if mode == "pow2" else Q.FREE
    dy_bits, x_bits = _bits(rng, t, nout), _bits(rng, t, kin)
    say(f"[sweep] wgrad {nout}x{kin} over {t} tokens acc={acc} scales={mode}")
    dy_c, dy_s = fp8q.quantize_act(_padded(dy_bits, rng), tile_axis="token_t", scale_mode=mode)
    x_c, x_s = fp8q.quantize_act(_padded(x_bits, rng), tile_axis="token_t", scale_mode=mode)
    ody_c, ody_s = Q.quantize_token_t(dy_bits, qm)
    ox_c, ox_s = Q.quantize_token_t(x_bits, qm)
    assert_codes_equal(host_codes(dy_c), ody_c, "dY codes")
    assert_scales_equal(host(dy_s), ody_s, "dY scales")
    assert_codes_equal(host_codes(x_c), ox_c, "X codes")
    assert_scales_equal(host(x_s), ox_s, "X scales")
    dw = host(fp8q.wgrad(dy_c.contiguous(), dy_s, x_c.contiguous(), x_s, acc=acc)).astype(np.float64)
    ref, s = G.wgrad(ody_c, ody_s, ox_c, ox_s)
    _accept(dw, ref, s, False, f"wgrad {nout}x{kin}x{t} {acc}")
