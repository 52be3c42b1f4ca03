"""GPU parity of the block-scaled GEMMs against the oracle.

Acceptance (both BF16-out and FP32-out): |gpu - oracle| <= 1e-5 * S + 1e-6
per element, S = sum_k |a_k * b_k| of the dequantized operands; for BF16
output the GPU value must be the RNE rounding of some float32 within that
tolerance.  Operands are quantized by the oracle on the host and the same
codes are given to both sides.

Shapes: the tiny linear (every element), ragged M/N/K and small cases (each
on both tilings of the dense float32-grade GEMM: 32 x 32 split-K tiles and
256-wide tiles, chosen with fp8q_set_gemm_small_limit), the
dense expert up-projection 4096 x 4096 x 7168 (sampled elements and full
rows), the MoE grouped GEMM with an empty expert, and the Wgrad 2048 x 7168
over 16384 tokens (sampled).  Closed forms: selector weights give an exactly
representable result; zero scales give exact zeros; K = 0 writes zeros.
"""

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q
from oracle import e4m3, gemm as G, quantize as Q
from tests import fp8_unit_model as unit
import synth
from tests.gpu_util import dev, host, host_bf16_bits, moe_operands, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _accept(c_dev, c_ref, s_ref, what):
    if c_dev.dtype == torch.bfloat16:
        got = host_bf16_bits(c_dev)
        ok = G.accept_bf16(got, c_ref, s_ref)
        gotv = e4m3.bf16_bits_to_f64(got)
    else:
        gotv = host(c_dev).astype(np.float64)
        ok = G.accept_f32(gotv, c_ref, s_ref)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; first {tuple(i)}: "
                             f"gpu {gotv[tuple(i)]!r} oracle {c_ref[tuple(i)]!r} S {s_ref[tuple(i)]!r}")


@pytest.fixture(params=["split_k_32x32", "tiles_256"])
def tiling(request):
    """Runs the test with the dense float32-grade GEMM forced onto one tiling:
    32 x 32 output tiles with the K blocks split over four waves, or 256-wide
    tiles over the whole of K; the library default is restored afterwards."""
    prev = fp8q.set_gemm_small_limit(1 << 62 if request.param == "split_k_32x32" else 0)
    yield request.param
    fp8q.set_gemm_small_limit(prev)


def _operands(a_bits, w_bits):
    a_c, a_s = Q.quantize_rows(a_bits)
    w_c, w_s = Q.quantize_blocks(w_bits)
    return a_c, a_s, w_c, w_s


def _run_dense(a_c, a_s, w_c, w_s, out_dtype):
    return fp8q.gemm(dev(a_c), dev(a_s), dev(w_c), dev(w_s), out_dtype=out_dtype)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_linear_every_element(out_dtype, tiling):
    d = synth.tiny_linear()
    a_c, a_s, w_c, w_s = _operands(d["a"], d["w"])
    say(f"[gemm] tiny linear 128x256x512 {out_dtype} {tiling}")
    c = _run_dense(a_c, a_s, w_c, w_s, out_dtype)
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    _accept(c, ref, s, "tiny linear")


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 5, 256), (17, 130, 384), (300, 202, 640),
                                   (256, 256, 1024), (513, 257, 128), (64, 1000, 256)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(m, n, k, out_dtype, tiling):
    rng = np.random.default_rng(m * 31 + n * 7 + k)
    a = synth.bf16_rne((rng.standard_normal((m, k)) * np.exp2(rng.integers(-3, 4, (m, k)))).astype(np.float32))
    w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    a_c, a_s, w_c, w_s = _operands(a, w)
    say(f"[gemm] ragged {m}x{n}x{k} {out_dtype} {tiling}")
    c = _run_dense(a_c, a_s, w_c, w_s, out_dtype)
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    _accept(c, ref, s, f"ragged {m}x{n}x{k}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_output_row_stride_and_untouched_padding(out_dtype, tiling):
    d = synth.tiny_linear()
    a_c, a_s, w_c, w_s = _operands(d["a"], d["w"])
    # a row stride of 262 elements is not a multiple of 4: element-wise stores
    for ld in (264, 262):
        out = torch.full((128, ld), float("nan"), dtype=out_dtype, device="cuda:0")
        say(f"[gemm] strided output ld={ld} {out_dtype} {tiling}")
        fp8q.gemm(dev(a_c), dev(a_s), dev(w_c), dev(w_s), out=out[:, :256])
        ref, s = G.gemm(a_c, a_s, w_c, w_s)
        _accept(out[:, :256], ref, s, f"strided output ld={ld}")
        assert torch.isnan(out[:, 256:]).all()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mid_size_every_element(out_dtype, tiling):
    """1000 x 1500 x 2560 (ragged in M and N; 20 K blocks, five per wave of
    the split-K tiling), activations with 0.1% outliers x100 as in the dense
    up-projection: every element against the oracle, and a second launch
    bit-identical to the first (the split-K sum has a fixed order)."""
    rng = np.random.default_rng(11)
    m, n, k = 1000, 1500, 2560
    a = rng.standard_normal((m, k)).astype(np.float32)
    hit = rng.choice(m * k, size=m * k // 1000, replace=False)
    a.reshape(-1)[hit] *= np.float32(100.0)
    a = synth.bf16_rne(a)
    w = synth.bf16_rne((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    a_c, a_s, w_c, w_s = _operands(a, w)
    say(f"[gemm] mid size {m}x{n}x{k} {out_dtype} {tiling}")
    ops = (dev(a_c), dev(a_s), dev(w_c), dev(w_s))
    c = fp8q.gemm(*ops, out_dtype=out_dtype)
    ref, s = G.gemm(a_c, a_s, w_c, w_s)
    _accept(c, ref, s, f"mid size {tiling}")
    c2 = fp8q.gemm(*ops, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16) if out_dtype == torch.bfloat16 else c.view(torch.int32),
                       c2.view(torch.int16) if out_dtype == torch.bfloat16 else c2.view(torch.int32))


def test_selector_weights_are_exact(tiling):
    """One nonzero weight code (+-1.0) per row per 128-block: C is a sum of
    K/128 scaled activation values, exactly computable; with power-of-two
    scales every term is exact in float32 and so is the GPU result."""
    rng = np.random.default_rng(8)
    m, n, k = 64, 256, 512
    # codes 0.5 .. 7.5 and scales 2^-2 .. 2^2: every partial sum stays within
    # 24 significant bits, so float32 accumulation in any order is exact
    a_c = rng.integers(0x30, 0x50, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    a_s = np.exp2(rng.integers(-2, 3, (m, k // 128))).astype(np.float32)
    w_c = np.zeros((n, k), np.uint8)
    for j in range(n):
        for b in range(k // 128):
            w_c[j, b * 128 + rng.integers(0, 128)] = 0x38 | (0x80 * rng.integers(0, 2))
    w_s = np.exp2(rng.integers(-2, 3, (2, k // 128))).astype(np.float32)
    say(f"[gemm] selector weights {tiling}")
    c = host(_run_dense(a_c, a_s, w_c, w_s, torch.float32)).astype(np.float64)
    ref, _ = G.gemm(a_c, a_s, w_c, w_s)
    assert np.array_equal(c, ref)


def test_zero_scales_and_k_zero(tiling):
    d = synth.tiny_linear()
    a_c, a_s, w_c, w_s = _operands(d["a"], d["w"])
    a_s = a_s.copy()
    a_s[7, :] = 0
    say("[gemm] zero scales")
    c = host(_run_dense(a_c, a_s, w_c, w_s, torch.float32))
    assert not c[7].any()
    say("[gemm] K = 0")
    out = torch.full((5, 16), 3.0, dtype=torch.float32, device="cuda:0")
    empty_c = torch.empty((5, 0), dtype=torch.uint8, device="cuda:0")
    empty_w = torch.empty((16, 0), dtype=torch.uint8, device="cuda:0")
    es = torch.empty((5, 0), dtype=torch.float32, device="cuda:0")
    ew = torch.empty((1, 0), dtype=torch.float32, device="cuda:0")
    fp8q.gemm(empty_c, es, empty_w, ew, out=out)
    assert not host(out).any()


def test_dense_up_projection_sampled():
    d = synth.dense_up()
    a_c, a_s, w_c, w_s = _operands(d["a"], d["w"])
    say("[gemm] dense up-projection 4096x4096x7168 bf16")
    c = _run_dense(a_c, a_s, w_c, w_s, torch.bfloat16)
    cb = host_bf16_bits(c)
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, 4096, 6000), np.repeat([0, 2047, 4095], 4096)])
    cols = np.concatenate([rng.integers(0, 4096, 6000), np.tile(np.arange(4096), 3)])
    for lo in range(0, rows.size, 4096):
        r, q = rows[lo:lo + 4096], cols[lo:lo + 4096]
        ref, s = G.gemm_at(a_c, a_s, w_c, w_s, r, q)
        ok = G.accept_bf16(cb[r, q], ref, s)
        assert ok.all(), f"dense sampled chunk {lo}: {int((~ok).sum())} bad"
    # every element of whole 256 x 256 output tiles (one workgroup each): the
    # corners and one tile of each XCD's tile range (XCD x runs tile rows
    # 4(x//2)..+3 and tile columns 8(x%2)..+7 of the 16 x 16 tile grid)
    tiles = [(0, 0), (15, 15), (0, 15), (15, 0)] + [(4 * (x // 2) + x % 4, 8 * (x % 2) + x) for x in range(8)]
    for tm, tn in tiles:
        r0, c0 = 256 * tm, 256 * tn
        ref, s = G.gemm(a_c[r0:r0 + 256], a_s[r0:r0 + 256], w_c[c0:c0 + 256], w_s[c0 // 128:c0 // 128 + 2])
        ok = G.accept_bf16(cb[r0:r0 + 256, c0:c0 + 256], ref, s)
        assert ok.all(), f"dense tile ({tm}, {tn}): {int((~ok).sum())} of 65536 bad"


def _grouped_case(tokens, hidden, inter, with_down):
    d = synth.moe_grouped(tokens=tokens, hidden=hidden, inter=inter)
    x_c, x_s = Q.quantize_rows(d["x"])
    a_c, a_s = x_c[d["gather"]], x_s[d["gather"]]  # quantize, then gather by expert
    def blocks(w):
        q = [Q.quantize_blocks(w[i]) for i in range(w.shape[0])]
        return np.stack([c for c, _ in q]), np.stack([s for _, s in q])

    out = [(a_c, a_s) + blocks(d["w_up"])]
    if with_down:
        h_c, h_s = Q.quantize_rows(d["h"])
        out.append((h_c, h_s) + blocks(d["w_down"]))
    return d, out


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_small_every_element(out_dtype):
    d, cases = _grouped_case(tokens=512, hidden=384, inter=256, with_down=True)
    offs = d["offsets"]
    assert (np.diff(offs) == 0).any()
    for name, (a_c, a_s, wc, ws) in zip(("up", "down"), cases):
        rows = a_c.shape[0]
        say(f"[gemm] grouped small {name} rows={rows} N={wc.shape[1]} K={wc.shape[2]} {out_dtype}")
        out = torch.full((rows + 3, wc.shape[1]), float("nan"), dtype=out_dtype, device="cuda:0")
        cap = torch.cat([dev(a_c), torch.zeros((3, a_c.shape[1]), dtype=torch.uint8, device="cuda:0")])
        cap_s = torch.cat([dev(a_s), torch.zeros((3, a_s.shape[1]), dtype=torch.float32, device="cuda:0")])
        fp8q.grouped_gemm(cap, cap_s, dev(offs), dev(wc), dev(ws), out=out)
        ref, s = G.grouped_gemm(a_c, a_s, offs, wc, ws)
        _accept(out[:rows], ref, s, f"grouped {name}")
        assert torch.isnan(out[rows:].float()).all()  # rows beyond offsets[G] untouched


def test_grouped_moe_one_gpu_share_sampled():
    d, cases = moe_operands()
    offs = d["offsets"]
    say(f"[gemm] MoE grouped 16 experts, M per expert {d['counts'].tolist()}")
    for name, (a_c, a_s, wc, ws) in cases.items():
        c = fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws), out_dtype=torch.bfloat16)
        cb = host_bf16_bits(c)
        rng = np.random.default_rng(2)
        for gi in range(len(offs) - 1):
            lo, hi = int(offs[gi]), int(offs[gi + 1])
            if hi == lo:
                continue
            rows = np.concatenate([rng.integers(lo, hi, 300), [lo, hi - 1]])
            cols = np.concatenate([rng.integers(0, wc.shape[1], 300), [0, wc.shape[1] - 1]])
            ref, s = G.gemm_at(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi], rows - lo, cols)
            ok = G.accept_bf16(cb[rows, cols], ref, s)
            assert ok.all(), f"grouped {name} expert {gi}: {int((~ok).sum())} bad"
            # every element of the expert's first output tile and of its last
            # (ragged in M unless the expert's rows are a multiple of 256;
            # both N, 4096 and 7168, are multiples of 256)
            n = wc.shape[1]
            last_m = lo + ((hi - lo - 1) // 256) * 256
            for r0, c0 in {(lo, 0), (last_m, n - 256)}:
                r1 = min(r0 + 256, hi)
                ref, s = G.gemm(a_c[r0:r1], a_s[r0:r1], wc[gi][c0:c0 + 256], ws[gi][c0 // 128:c0 // 128 + 2])
                ok = G.accept_bf16(cb[r0:r1, c0:c0 + 256], ref, s)
                assert ok.all(), f"grouped {name} expert {gi} tile rows {r0}..{r1}: {int((~ok).sum())} bad"


def test_grouped_offsets_past_rows_cap_are_clamped():
    """A routing table whose last offset runs past rows_cap: the kernel clamps
    each group's rows to [0, rows_cap], so the groups inside are computed as
    usual, the one that straddles rows_cap is cut there, and nothing is read
    or written beyond rows_cap (guard rows of the output stay NaN)."""
    d, cases = _grouped_case(tokens=256, hidden=256, inter=128, with_down=False)
    _, _, wc, ws = cases[0]
    g, n, k = wc.shape[0], wc.shape[1], wc.shape[2]
    rows_cap = 300
    bounds = [0, 100, 250] + [400] * (g - 2)  # offsets[G] = 400 > rows_cap
    offs = np.array(bounds, dtype=np.int32)
    rng = np.random.default_rng(5)
    a_bits = synth.bf16_rne(rng.standard_normal((rows_cap, k)).astype(np.float32))
    a_c, a_s = Q.quantize_rows(a_bits)
    say(f"[gemm] grouped, offsets {bounds[:4]}... past rows_cap={rows_cap}")
    full = torch.full((rows_cap + 64, n), float("nan"), dtype=torch.float32, device="cuda:0")
    fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws), out=full[:rows_cap])
    got = host(full)
    assert np.isnan(got[rows_cap:]).all(), "rows beyond rows_cap were written"
    for gi, (lo, hi) in enumerate([(0, 100), (100, 250), (250, rows_cap)]):
        ref, s = G.gemm(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi])
        ok = G.accept_f32(got[lo:hi].astype(np.float64), ref, s)
        assert ok.all(), f"group {gi}: {int((~ok).sum())} bad"


def test_grouped_equals_dense_per_group():
    """The grouped GEMM and the dense GEMM on 256-wide tiles run the same K
    loop, so each group's rows are bit-identical to a dense call on them (the
    32 x 32 split-K tiling sums in another order and is held to the oracle
    instead, above)."""
    d, cases = _grouped_case(tokens=256, hidden=256, inter=128, with_down=False)
    a_c, a_s, wc, ws = cases[0]
    offs = d["offsets"]
    say("[gemm] grouped == dense per group")
    cg = host(fp8q.grouped_gemm(dev(a_c), dev(a_s), dev(offs), dev(wc), dev(ws), out_dtype=torch.float32))
    prev = fp8q.set_gemm_small_limit(0)
    try:
        for gi in range(len(offs) - 1):
            lo, hi = int(offs[gi]), int(offs[gi + 1])
            if hi > lo:
                cd = host(_run_dense(a_c[lo:hi], a_s[lo:hi], wc[gi], ws[gi], torch.float32))
                assert np.array_equal(cg[lo:hi], cd), gi
    finally:
        fp8q.set_gemm_small_limit(prev)


def _wgrad_operands(dy_bits, x_bits):
    dy_c, dy_s = Q.quantize_token_t(dy_bits)
    x_c, x_s = Q.quantize_token_t(x_bits)
    return dy_c, dy_s, x_c, x_s


@pytest.mark.parametrize("t,nout,kin", [(128, 1, 1), (384, 300, 260), (1024, 256, 512)])
def test_wgrad_small_every_element(t, nout, kin):
    rng = np.random.default_rng(t + nout + kin)
    dy = synth.bf16_rne(rng.standard_normal((t, nout)).astype(np.float32))
    x = synth.bf16_rne(rng.standard_normal((t, kin)).astype(np.float32))
    ops = _wgrad_operands(dy, x)
    say(f"[gemm] wgrad T={t} {nout}x{kin}")
    dw = fp8q.wgrad(*[dev(o) for o in ops])
    ref, s = G.wgrad(*ops)
    _accept(dw, ref, s, "wgrad small")


@pytest.mark.parametrize("acc", ["fp32", "fp8_mfma"])
def test_wgrad_tile_widths(acc):
    """The weight gradient picks 224-column tiles when that fills more CUs for
    less time (most shapes here, and the 2048 x 7168 workload) and 256-column
    tiles otherwise: 2048 x 8192 makes 256 tiles of 256 columns (one wave on
    256 CUs) but 296 of 224.  Every element of that case (FP32-grade), or a
    sample covering every row and column (FP8 unit, against the unit model)."""
    from oracle import accum
    from tests.test_gpu_native import _accept_model
    rng = np.random.default_rng(8192)
    t, nout, kin = 256, 2048, 8192
    dy = synth.bf16_rne(rng.standard_normal((t, nout)).astype(np.float32))
    x = synth.bf16_rne(rng.standard_normal((t, kin)).astype(np.float32))
    ops = _wgrad_operands(dy, x)
    say(f"[gemm] wgrad T={t} {nout}x{kin} (256-column tiles) acc={acc}")
    dw = fp8q.wgrad(*[dev(o) for o in ops], acc=acc)
    if acc == "fp32":
        ref, s = G.wgrad(*ops)
        _accept(dw, ref, s, "wgrad 256-column tiles")
        return
    rows = np.concatenate([np.arange(nout), rng.integers(0, nout, kin), rng.integers(0, nout, 3000)])
    cols = np.concatenate([rng.integers(0, kin, nout), np.arange(kin), rng.integers(0, kin, 3000)])
    got = dw[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()]
    ref, s, tt = unit.gemm_at_mfma(ops[0], ops[1], ops[2], ops[3], rows, cols, w_block_rows=False)
    _accept_model(got, ref, s, tt, "wgrad 256-column tiles, FP8 unit")


def test_wgrad_full_sampled():
    d = synth.wgrad()
    ops = _wgrad_operands(d["dy"], d["x"])
    say("[gemm] wgrad 2048x7168 over 16384 tokens")
    dw = host(fp8q.wgrad(*[dev(o) for o in ops])).astype(np.float64)
    rng = np.random.default_rng(3)
    rows = np.concatenate([rng.integers(0, 2048, 4000), np.zeros(7168, np.int64)])
    cols = np.concatenate([rng.integers(0, 7168, 4000), np.arange(7168)])
    for lo in range(0, rows.size, 2048):
        r, q = rows[lo:lo + 2048], cols[lo:lo + 2048]
        ref, s = G.gemm_at(ops[0], ops[1], ops[2], ops[3], r, q, w_block_rows=False)
        ok = G.accept_f32(dw[r, q], ref, s)
        assert ok.all(), f"wgrad chunk {lo}: {int((~ok).sum())} bad"
    # every element of whole output tiles: the launch uses 256 x 224 tiles
    # here (8 x 32 of them); first, last and four more spread over the grid
    for tm, tn in [(0, 0), (7, 31), (3, 5), (4, 16), (1, 30), (6, 11)]:
        r0, c0 = 256 * tm, 224 * tn
        ref, s = G.wgrad(ops[0][r0:r0 + 256], ops[1][r0:r0 + 256], ops[2][c0:c0 + 224], ops[3][c0:c0 + 224])
        ok = G.accept_f32(dw[r0:r0 + 256, c0:c0 + 224], ref, s)
        assert ok.all(), f"wgrad tile ({tm}, {tn}): {int((~ok).sum())} bad"


def test_gemm_deterministic():
    d = synth.tiny_linear()
    ops = [dev(o) for o in _operands(d["a"], d["w"])]
    say("[gemm] determinism")
    c1 = fp8q.gemm(*ops, out_dtype=torch.float32)
    c2 = fp8q.gemm(*ops, out_dtype=torch.float32)
    assert torch.equal(c1, c2)
