"""Bench of the fine-grained FP8 linear-layer hot path on one MI355X.

One step = one pass of the path over the dense expert up-projection
(A BF16 4096 x 7168 with 0.1% outliers x100, W BF16 4096 x 7168 ~N(0, 0.02)):
1x128 online max-abs quantization of A and 128x128 quantization of W (one
launch, fp8q_quantize_linear), then the block-scaled FP8 GEMM to BF16
C[4096, 4096] -- all in libfp8q.so.
Inputs are generated on the host (seeded), copied to HBM once, and are
resident before the timed region starts.

Prints one JSON line:
  value      = whole-step throughput, 2*M*N*K / step time (TFLOP/s)
  kernels    = per-kernel average durations from HIP events on the launch
               stream around --steps back-to-back launches of that kernel,
               with GB/s or TFLOP/s and the fraction of the MI355X roofline
  *_after_cache_flush = the step's GEMM and quantizer as single launches,
               each after a 1 GiB write that evicts the caches (median, min)
  roofline   = the dominant kernel (the GEMM) against the dense FP8 MFMA peak
  cpu_baseline = the oracle timed on the host on a bounded sample

    python bench.py [--gpus 1] [--steps 200] [--warmup 400] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, N, K = 4096, 4096, 7168
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
METRIC = "block-scaled FP8 GEMM TFLOP/s + quantize GB/s, % of MI355X roofline"

# algorithmic bytes: BF16 read + code write + one float32 scale per tile
ACT_BYTES = M * K * 2 + M * K + M * (K // 128) * 4
WGT_BYTES = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
GEMM_FLOP = 2.0 * M * N * K
# HBM traffic of one dense GEMM launch (acc=FP32) from rocprofv3 counters
# (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, calibrated on a 256 MiB copy) for
# the kernel as it stands; None until re-measured after a kernel change
GEMM_TRAFFIC_BYTES = 217_230_000


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the GPU needs tens of milliseconds of load to reach its steady clock:
    # the default warm-up (400 steps, ~90 ms, untimed) runs past that ramp,
    # and the timed region is 200 steps (~45 ms)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (torch) --steps times; used to "
                        "scale the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run")
    return p.parse_args()


def copy_calibration(steps):
    """A plain copy of known size: 256 MiB read + 256 MiB written per launch."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "us": round(us, 2),
                      "GB/s": round(2 * n / (us * 1e-6) / 1e9, 1)}), flush=True)


def cpu_baseline():
    """The oracle (as it stands) on a bounded sample of the same workload:
    quantize 1024 rows of A and 1024 rows of W, then the block-scaled GEMM of
    those rows (1024 x 1024 x 7168).  Rate = GEMM FLOPs / total time."""
    import threadpoolctl
    from oracle import gemm as G, quantize as Q
    import synth
    d = synth.dense_up()
    rows = 1024
    a, w = np.ascontiguousarray(d["a"][:rows]), np.ascontiguousarray(d["w"][:rows])
    t0 = time.perf_counter()
    a_c, a_s = Q.quantize_rows(a)
    w_c, w_s = Q.quantize_blocks(w)
    t1 = time.perf_counter()
    G.gemm(a_c, a_s, w_c, w_s)
    t2 = time.perf_counter()
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    flop = 2.0 * rows * rows * K
    return {"value": flop / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"A rows 0..{rows - 1} and W rows 0..{rows - 1} of the 4096x4096x7168 workload: "
                      f"quantize ({t1 - t0:.2f} s) + GEMM {rows}x{rows}x{K} ({t2 - t1:.2f} s), "
                      f"rate = GEMM FLOPs / total"}


def quantize_only_rates(torch, fp8q, lib, stream, reps):
    """Quantizer bandwidth at the quantize-only sizes: activations 16384 x 7168
    (standard Student-t(3)) in free and power-of-two modes, weights 7168 x 18432
    (~N(0, 0.02)).  HIP events around `reps` launches alternating over two
    input/output sets (each set is larger than the Infinity Cache)."""
    import synth
    dev = torch.device("cuda:0")
    out = {}
    act = synth.quant_only_act()
    rows, cols = act.shape
    xs = [torch.from_numpy(act.view(np.int16)).view(torch.bfloat16).to(dev)]
    xs.append(xs[0].clone())
    cs = [torch.empty((rows, cols), dtype=torch.uint8, device=dev) for _ in range(2)]
    ss = torch.empty((rows, cols // 128), dtype=torch.float32, device=dev)
    abytes = rows * cols * 3 + rows * (cols // 128) * 4
    for mode_name, mode in (("free", fp8q.SCALE_FREE), ("pow2", fp8q.SCALE_POW2)):
        def fn(i):
            return lib.fp8q_quantize_act(xs[i & 1].data_ptr(), rows, cols, cols, fp8q.TILE_ROW, mode,
                                         cs[i & 1].data_ptr(), cols, ss.data_ptr(), stream.cuda_stream)
        burst = _burst_us(torch, stream, fn)
        us = _event_us(torch, stream, fn, reps)
        out[f"act_16384x7168_{mode_name}"] = {"us": round(us, 2), "GB/s": round(abytes / us / 1e3, 1),
                                              "frac_hbm": round(abytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                              "bytes": abytes, "us_first_20_after_idle": round(burst, 2),
                                              "frac_hbm_first_20_after_idle":
                                                  round(abytes / burst / 1e3 / HBM_PEAK_GBS, 4)}
    del xs, cs, ss
    wt = synth.quant_only_weight()
    n, k = wt.shape
    ws = [torch.from_numpy(wt.view(np.int16)).view(torch.bfloat16).to(dev)]
    ws.append(ws[0].clone())
    cs = [torch.empty((n, k), dtype=torch.uint8, device=dev) for _ in range(2)]
    ss = torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev)
    wbytes = n * k * 3 + (n // 128) * (k // 128) * 4

    def fw(i):
        return lib.fp8q_quantize_weight(ws[i & 1].data_ptr(), n, k, k, fp8q.SCALE_FREE, cs[i & 1].data_ptr(),
                                        k, ss.data_ptr(), stream.cuda_stream)
    burst = _burst_us(torch, stream, fw)
    us = _event_us(torch, stream, fw, reps)
    out["weight_7168x18432"] = {"us": round(us, 2), "GB/s": round(wbytes / us / 1e3, 1),
                                "frac_hbm": round(wbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": wbytes,
                                "us_first_20_after_idle": round(burst, 2),
                                "frac_hbm_first_20_after_idle": round(wbytes / burst / 1e3 / HBM_PEAK_GBS, 4)}
    return out


def _roofline(flop, nbytes, us):
    """Time at the roofline max(flop / FP8 peak, bytes / HBM peak) and the
    fraction of it reached in `us`."""
    t = max(flop / (FP8_PEAK_TFLOPS * 1e6), nbytes / (HBM_PEAK_GBS * 1e3))
    return {"us": round(us, 2), "TFLOP/s": round(flop / us / 1e6, 1), "GB/s": round(nbytes / us / 1e3, 1),
            "flop": flop, "bytes": nbytes, "roofline_us": round(t, 2), "frac_roofline": round(t / us, 4),
            "bound": "mfma" if flop / (FP8_PEAK_TFLOPS * 1e6) >= nbytes / (HBM_PEAK_GBS * 1e3) else "hbm"}


def moe_rates(torch, fp8q, lib, stream, reps):
    """One GPU's share of the MoE layer: 8192 tokens routed top-8 over 256
    experts (Zipf(1.1) popularity), 16 hosted experts, one of them empty.
    Tokens are quantized once (1x128), then their codes and scales are
    gathered by expert (FP8 dispatch gather); grouped up-projection
    7168 -> 4096 and grouped down-projection 2048 -> 7168, BF16 out; the
    SwiGLU between them fused with the 1x128 quantization of its output; and
    the whole expert FFN forward (gather, up, SwiGLU + quantize, down) as one
    timed pass."""
    import synth
    dev = torch.device("cuda:0")
    d = synth.moe_grouped()
    G = len(d["counts"])
    rows = int(d["counts"].sum())
    K_UP = d["x"].shape[1]

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    x = bf(d["x"])
    xq, xs = fp8q.quantize_act(x)
    gather = torch.from_numpy(d["gather"].astype(np.int32)).to(dev)
    a_up, s_up = fp8q.gather_rows(xq, xs, gather)
    off = torch.from_numpy(d["offsets"]).to(dev)
    hq, hs = fp8q.quantize_act(bf(d["h"]))
    out = {"experts": G, "rows_per_expert": [int(v) for v in d["counts"]], "rows": rows}

    # FP8 dispatch gather of the hosted rows; the timing rotates over five
    # copies of the quantized tokens (more than the 256 MB Infinity Cache)
    nb_up = K_UP // 128
    srcs = [(xq, xs)] + [fp8q.quantize_act(x) for _ in range(4)]

    def fg_from(i):
        q, sc = srcs[i % len(srcs)]
        return lib.fp8q_gather_rows(q.data_ptr(), q.shape[0], K_UP, q.stride(0), sc.data_ptr(),
                                    gather.data_ptr(), rows, a_up.data_ptr(), a_up.stride(0), s_up.data_ptr(),
                                    stream.cuda_stream)
    us = _event_us(torch, stream, fg_from, reps)
    del srcs

    def fg(i):
        return lib.fp8q_gather_rows(xq.data_ptr(), xq.shape[0], K_UP, xq.stride(0), xs.data_ptr(),
                                    gather.data_ptr(), rows, a_up.data_ptr(), a_up.stride(0), s_up.data_ptr(),
                                    stream.cuda_stream)
    gbytes = 2 * rows * (K_UP + nb_up * 4) + rows * 4
    out["dispatch_gather_fp8"] = {"us": round(us, 2), "GB/s": round(gbytes / us / 1e3, 1),
                                  "frac_hbm": round(gbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": gbytes}

    # SwiGLU + 1x128 quantization of the up-projection output shape, inputs
    # rotated over ten copies (more than the Infinity Cache)
    inter = d["w_down"].shape[2]
    sx0 = bf(synth.swiglu_input(rows=rows, inter=inter))
    sxs = [sx0] + [sx0.clone() for _ in range(9)]
    sq = torch.empty((rows, inter), dtype=torch.uint8, device=dev)
    ss = torch.empty((rows, inter // 128), dtype=torch.float32, device=dev)
    cq = torch.empty((rows, 2 * inter), dtype=torch.uint8, device=dev)
    cs = torch.empty((rows, 2 * inter // 128), dtype=torch.float32, device=dev)
    for name, cache in (("swiglu_quantize", False), ("swiglu_quantize_with_pow2_cache", True)):
        def fs(i, cache=cache):
            return lib.fp8q_swiglu_quantize(sxs[i % len(sxs)].data_ptr(), rows, inter, 2 * inter, fp8q.SCALE_FREE,
                                            sq.data_ptr(), inter, ss.data_ptr(), fp8q.SCALE_POW2,
                                            cq.data_ptr() if cache else None, 2 * inter,
                                            cs.data_ptr() if cache else None, stream.cuda_stream)
        us = _event_us(torch, stream, fs, reps)
        sbytes = rows * 2 * inter * 2 + rows * inter + rows * (inter // 128) * 4
        if cache:
            sbytes += rows * 2 * inter + rows * (2 * inter // 128) * 4
        out[name] = {"us": round(us, 2), "GB/s": round(sbytes / us / 1e3, 1),
                     "frac_hbm": round(sbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": sbytes}
    del sxs, sx0, cq, cs

    weights = {}
    for name, wname, in_a, in_s in (("up_7168x4096", "w_up", a_up, s_up), ("down_2048x7168", "w_down", hq, hs)):
        wb = bf(d[wname])
        g, n, k = wb.shape
        wq, ws = fp8q.quantize_weight(wb.view(g * n, k))
        del wb
        weights[wname] = (wq, ws, n, k)
        c = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
        for acc_name, acc in (("", fp8q.ACC_FP32), ("_fp8_mfma", fp8q.ACC_FP8_MFMA)):
            out[name + acc_name] = _grouped_rate(torch, lib, stream, reps, d["counts"], in_a, in_s, off, G, rows,
                                                 wq, ws, n, k, c, acc, fp8q)
        del c

    # expert FFN forward, default accumulation: dispatch gather -> up ->
    # SwiGLU + quantize -> down
    wq_u, ws_u, n_u, k_u = weights["w_up"]
    wq_d, ws_d, n_d, k_d = weights["w_down"]
    up_out = torch.empty((rows, n_u), dtype=torch.bfloat16, device=dev)
    y = torch.empty((rows, n_d), dtype=torch.bfloat16, device=dev)

    def ffn(i):
        st = fg(i)
        st = st or lib.fp8q_grouped_gemm_ex(a_up.data_ptr(), s_up.data_ptr(), off.data_ptr(), G, rows,
                                         wq_u.data_ptr(), ws_u.data_ptr(), n_u, k_u, fp8q.OUT_BF16,
                                         fp8q.ACC_FP32, up_out.data_ptr(), n_u, stream.cuda_stream)
        st = st or lib.fp8q_swiglu_quantize(up_out.data_ptr(), rows, inter, n_u, fp8q.SCALE_FREE,
                                            sq.data_ptr(), inter, ss.data_ptr(), fp8q.SCALE_POW2, None, 0,
                                            None, stream.cuda_stream)
        st = st or lib.fp8q_grouped_gemm_ex(sq.data_ptr(), ss.data_ptr(), off.data_ptr(), G, rows,
                                         wq_d.data_ptr(), ws_d.data_ptr(), n_d, k_d, fp8q.OUT_BF16,
                                         fp8q.ACC_FP32, y.data_ptr(), n_d, stream.cuda_stream)
        return st
    us = _event_us(torch, stream, ffn, reps)
    flop = 2.0 * rows * (n_u * k_u + n_d * k_d)
    out["expert_ffn_forward"] = {"us": round(us, 2), "TFLOP/s": round(flop / us / 1e6, 1), "flop": flop,
                                 "steps": "dispatch gather, grouped up GEMM, SwiGLU + quantize, grouped down GEMM"}
    return out


def _grouped_rate(torch, lib, stream, reps, counts, in_a, in_s, off, G, rows, wq, ws, n, k, c, acc, fp8q):
    """Grouped GEMM time for one accumulation mode, with the whole-kernel and
    the per-expert roofline."""
    def fn(i):
        return lib.fp8q_grouped_gemm_ex(in_a.data_ptr(), in_s.data_ptr(), off.data_ptr(), G, rows,
                                     wq.data_ptr(), ws.data_ptr(), n, k, fp8q.OUT_BF16, acc, c.data_ptr(),
                                     n, stream.cuda_stream)
    us = _event_us(torch, stream, fn, reps)
    flop = 2.0 * rows * n * k
    nbytes = G * n * k + (G * n // 128) * (k // 128) * 4 + rows * k + rows * (k // 128) * 4 + rows * n * 2
    r = _roofline(flop, nbytes, us)
    # sum over experts of each expert's own roofline time (a small
    # expert is bound by reading its weights)
    per = 0.0
    for m in counts:
        fe = 2.0 * int(m) * n * k
        be = n * k + (n // 128) * (k // 128) * 4 + int(m) * (k + (k // 128) * 4 + n * 2)
        per += max(fe / (FP8_PEAK_TFLOPS * 1e6), be / (HBM_PEAK_GBS * 1e3)) if m else 0.0
    r["per_expert_roofline_us"] = round(per, 2)
    return r


def wgrad_rates(torch, fp8q, lib, stream, reps):
    """Weight gradient over 16384 tokens: dY 16384 x 2048 and X 16384 x 7168
    (BF16 ~N(0,1)) quantized in 128-token x 1-feature tiles (codes written
    feature-major), then dW[2048, 7168] = dY^T X in FP32."""
    import synth
    dev = torch.device("cuda:0")
    d = synth.wgrad()
    out = {}
    q = {}
    for name, arr in (("dy", d["dy"]), ("x", d["x"])):
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
        tok, feat = t.shape
        codes = torch.empty((feat, tok), dtype=torch.uint8, device=dev)
        scales = torch.empty((feat, tok // 128), dtype=torch.float32, device=dev)

        def fn(i, t=t, tok=tok, feat=feat, codes=codes, scales=scales):
            return lib.fp8q_quantize_act(t.data_ptr(), tok, feat, feat, fp8q.TILE_TOKEN_T, fp8q.SCALE_FREE,
                                         codes.data_ptr(), tok, scales.data_ptr(), stream.cuda_stream)
        us = _event_us(torch, stream, fn, reps)
        nbytes = tok * feat * 3 + feat * (tok // 128) * 4
        out[f"quantize_{name}_token_t_{tok}x{feat}"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                                        "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                                        "bytes": nbytes}
        q[name] = (codes, scales, tok, feat)
        del t
    dyc, dys, T, nout = q["dy"]
    xc, xs, _, kin = q["x"]
    dw = torch.empty((nout, kin), dtype=torch.float32, device=dev)

    flop = 2.0 * nout * kin * T
    nbytes = (nout + kin) * T + (nout + kin) * (T // 128) * 4 + nout * kin * 4
    for acc_name, acc in (("", fp8q.ACC_FP32), ("_fp8_mfma", fp8q.ACC_FP8_MFMA)):
        def fg(i, acc=acc):
            return lib.fp8q_wgrad_ex(dyc.data_ptr(), dys.data_ptr(), xc.data_ptr(), xs.data_ptr(), nout, kin, T,
                                  acc, dw.data_ptr(), kin, stream.cuda_stream)
        us = _event_us(torch, stream, fg, reps)
        out[f"wgrad_{nout}x{kin}x{T}{acc_name}"] = _roofline(flop, nbytes, us)
    return out


def dgrad_rates(torch, fp8q, lib, stream, reps, w):
    """Activation gradient of the up-projection: the weight W [4096, 7168]
    quantized once into both orientations (one read, two code copies), then
    dX [4096, 7168] = dY [4096, 4096] . W (reduction over N = 4096), dY
    BF16 ~N(0,1) quantized in 1x128 tiles along N, BF16 out."""
    import synth
    dev = torch.device("cuda:0")
    n, k = w.shape
    m = 4096
    codes = torch.empty((n, k), dtype=torch.uint8, device=dev)
    scales = torch.empty((n // 128, k // 128), dtype=torch.float32, device=dev)
    codes_t = torch.empty((k, n), dtype=torch.uint8, device=dev)
    scales_t = torch.empty((k // 128, n // 128), dtype=torch.float32, device=dev)
    w2 = [w, w.clone()]

    def fq(i):
        return lib.fp8q_quantize_weight_t(w2[i & 1].data_ptr(), n, k, k, fp8q.SCALE_FREE, codes.data_ptr(), k,
                                          scales.data_ptr(), codes_t.data_ptr(), n, scales_t.data_ptr(),
                                          stream.cuda_stream)
    us_q = _event_us(torch, stream, fq, reps)
    qbytes = n * k * 4 + 2 * (n // 128) * (k // 128) * 4
    out = {"quantize_weight_both_orientations_4096x7168": {
        "us": round(us_q, 2), "GB/s": round(qbytes / us_q / 1e3, 1),
        "frac_hbm": round(qbytes / us_q / 1e3 / HBM_PEAK_GBS, 4), "bytes": qbytes}}
    rng = np.random.default_rng(21)
    dy = torch.from_numpy(synth.bf16_rne(rng.standard_normal((m, n)).astype(np.float32)).view(np.int16))
    dyq, dys = fp8q.quantize_act(dy.view(torch.bfloat16).to(dev))
    dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    flop = 2.0 * m * n * k
    nbytes = m * n + n * k + m * (n // 128) * 4 + (k // 128) * (n // 128) * 4 + m * k * 2
    for acc_name, acc in (("", fp8q.ACC_FP32), ("_fp8_mfma", fp8q.ACC_FP8_MFMA)):
        def fg(i, acc=acc):
            return lib.fp8q_gemm_ex(dyq.data_ptr(), dys.data_ptr(), codes_t.data_ptr(), scales_t.data_ptr(), m, k,
                                 n, fp8q.OUT_BF16, acc, dx.data_ptr(), k, stream.cuda_stream)
        out[f"dgrad_{m}x{k}x{n}{acc_name}"] = _roofline(flop, nbytes, _event_us(torch, stream, fg, reps))
    return out


def _burst_us(torch, stream, fn, reps=20):
    """Average of `reps` launches started after 200 ms without GPU work.  The
    HBM-bound kernels run at their full rate for the first ~1.5 ms of
    sustained load and slower after that (the GPU's power management; the
    sustained average is the figure the roofline fraction uses)."""
    torch.cuda.synchronize()
    time.sleep(0.2)
    return _event_us(torch, stream, fn, reps)


def flushed_launch_us(torch, stream, fn, reps=20):
    """Median and min of single launches, each after a 1 GiB buffer (more
    than the 256 MB Infinity Cache and every L2) has been written, with one
    HIP event pair per launch."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(reps):
        scratch.fill_(i & 0xFF)
        e0.record(stream)
        if fn() != 0:
            raise RuntimeError("fp8q call failed")
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    return float(np.median(times)), float(np.min(times))


def rocm_smi_clocks():
    """Current clocks reported by rocm-smi (read after the measurements), or
    None where it is not available.  rocm-smi is a Python script: it is run
    by this interpreter as a child process, not through its `env` shebang,
    so no process that has loaded a profiler's GPU library replaces itself
    with another program."""
    import shutil
    import subprocess
    try:
        smi = shutil.which("rocm-smi")
        if smi is None:
            return None
        target = os.path.realpath(smi)
        cmd = [sys.executable, target] if target.endswith(".py") else [smi]
        r = subprocess.run(cmd + ["--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        text = r.stdout[r.stdout.index("{"):]
        cards = json.loads(text)
        card = cards[sorted(cards)[0]]
        return {k.strip(" :"): v for k, v in card.items()}
    except Exception:
        return None


def _event_us(torch, stream, fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn(0)
    fn(1)
    e0.record(stream)
    for i in range(reps):
        if fn(i) != 0:
            raise RuntimeError("fp8q call failed")
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "fp8q runs on one GPU only (no multi-GPU path); --gpus must be 1"}))
        sys.exit(2)

    import torch
    import fine_grained_fp8_fp8q_amd as fp8q
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    fp8q.load_library()
    dev = torch.device("cuda:0")
    d = synth.dense_up(m=M, n=N, k=K)
    a = torch.from_numpy(d["a"].view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(d["w"].view(np.int16)).view(torch.bfloat16).to(dev)
    a_codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    w_codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    a_scales = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    w_scales = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    lib = fp8q.load_library()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def gemm():
        return lib.fp8q_gemm_ex(a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(), w_scales.data_ptr(),
                             M, N, K, fp8q.OUT_BF16, fp8q.ACC_FP32, c.data_ptr(), N, sp)

    def q_both():
        # both quantizers in one launch; outputs identical to fp8q_quantize_act +
        # fp8q_quantize_weight
        return lib.fp8q_quantize_linear(a.data_ptr(), M, K, K, fp8q.SCALE_FREE, a_codes.data_ptr(), K,
                                        a_scales.data_ptr(), w.data_ptr(), N, K, fp8q.SCALE_FREE,
                                        w_codes.data_ptr(), K, w_scales.data_ptr(), sp)

    def step():
        st = q_both() | gemm()
        if st != fp8q.OK:
            raise RuntimeError(f"fp8q call failed with status {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, nothing else on the stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_events = ev0.elapsed_time(ev1) / args.steps

    # per-kernel durations: HIP events on the launch stream around --steps
    # back-to-back launches of one kernel (an event record is a queue barrier
    # packet, so one pair per run keeps it out of the average).  The
    # quantizers rotate over ROT copies of their input and output (more than
    # the 256 MB Infinity Cache), so each launch streams from HBM as in the
    # step; the GEMM re-reads its 58 MB of codes, which in the step were just
    # written by the quantizers.
    ROT = 5
    a_rot = [a] + [a.clone() for _ in range(ROT - 1)]
    w_rot = [w] + [w.clone() for _ in range(ROT - 1)]
    ac_rot = [torch.empty_like(a_codes) for _ in range(ROT)]
    wc_rot = [torch.empty_like(w_codes) for _ in range(ROT)]

    def q_act_i(i):
        return lib.fp8q_quantize_act(a_rot[i % ROT].data_ptr(), M, K, K, fp8q.TILE_ROW, fp8q.SCALE_FREE,
                                     ac_rot[i % ROT].data_ptr(), K, a_scales.data_ptr(), sp)

    def q_wgt_i(i):
        return lib.fp8q_quantize_weight(w_rot[i % ROT].data_ptr(), N, K, K, fp8q.SCALE_FREE,
                                        wc_rot[i % ROT].data_ptr(), K, w_scales.data_ptr(), sp)

    def kernel_us(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(ROT):
            fn(i)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    qa_us = kernel_us(q_act_i)
    qw_us = kernel_us(q_wgt_i)

    def q_lin_i(i):
        return lib.fp8q_quantize_linear(a_rot[i % ROT].data_ptr(), M, K, K, fp8q.SCALE_FREE,
                                        ac_rot[i % ROT].data_ptr(), K, a_scales.data_ptr(), w_rot[i % ROT].data_ptr(),
                                        N, K, fp8q.SCALE_FREE, wc_rot[i % ROT].data_ptr(), K, w_scales.data_ptr(), sp)
    ql_us = kernel_us(q_lin_i)
    gemm_us = kernel_us(lambda i: gemm())
    gemm_f8_us = kernel_us(lambda i: lib.fp8q_gemm_ex(a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(),
                                                   w_scales.data_ptr(), M, N, K, fp8q.OUT_BF16,
                                                   fp8q.ACC_FP8_MFMA, c.data_ptr(), N, sp))
    # the hardware-scaled form needs power-of-two scales: the same inputs
    # quantized in that mode
    ap_codes, ap_scales = fp8q.quantize_act(a, scale_mode="pow2")
    wp_codes, wp_scales = fp8q.quantize_weight(w, scale_mode="pow2")
    gemm_f8s_us = kernel_us(lambda i: lib.fp8q_gemm_ex(ap_codes.data_ptr(), ap_scales.data_ptr(),
                                                    wp_codes.data_ptr(), wp_scales.data_ptr(), M, N, K,
                                                    fp8q.OUT_BF16, fp8q.ACC_FP8_MFMA_SCALED, c.data_ptr(), N, sp))
    del ap_codes, ap_scales, wp_codes, wp_scales
    # the GEMM with its output quantized in the epilogue (1x128 along N, the
    # FP8 input of a following layer) next to the unfused pair it replaces
    cq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    cqs = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
    gemm_q_us = kernel_us(lambda i: lib.fp8q_gemm_quantized(a_codes.data_ptr(), a_scales.data_ptr(),
                                                            w_codes.data_ptr(), w_scales.data_ptr(), M, N, K,
                                                            fp8q.ACC_FP32, fp8q.SCALE_FREE, cq.data_ptr(), N,
                                                            cqs.data_ptr(), sp))

    def unfused(i):
        st = gemm()
        return st or lib.fp8q_quantize_act(c.data_ptr(), M, N, N, fp8q.TILE_ROW, fp8q.SCALE_FREE, cq.data_ptr(),
                                           N, cqs.data_ptr(), sp)
    unfused_us = kernel_us(unfused)
    del cq, cqs
    flush_med_us, flush_min_us = flushed_launch_us(torch, stream, gemm)
    qflush_med_us, qflush_min_us = flushed_launch_us(torch, stream, lambda: q_lin_i(0))
    quant_only = quantize_only_rates(torch, fp8q, lib, stream, max(3, args.steps // 4))
    dg = dgrad_rates(torch, fp8q, lib, stream, max(3, args.steps // 4), w)
    del a_rot, w_rot, ac_rot, wc_rot
    moe = moe_rates(torch, fp8q, lib, stream, max(3, args.steps // 2))
    wg = wgrad_rates(torch, fp8q, lib, stream, max(3, args.steps // 4))
    qa_gbs = ACT_BYTES / (qa_us * 1e-6) / 1e9
    qw_gbs = WGT_BYTES / (qw_us * 1e-6) / 1e9
    gemm_tflops = GEMM_FLOP / (gemm_us * 1e-6) / 1e12
    gemm_f8_tflops = GEMM_FLOP / (gemm_f8_us * 1e-6) / 1e12
    value = GEMM_FLOP / (ms_step * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        # the same timed region seen by HIP events on the stream (excludes the
        # host's launch latency at its start and the wake-up at its end)
        "ms_per_step_stream_events": round(ms_step_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> f32 accumulate, bf16 in/out",
        "data": "synthetic (seeded): A ~N(0,1) with 0.1% entries x100, W ~N(0,0.02), BF16",
        "config": {"workload": "dense expert up-projection: quantize A 4096x7168 (1x128) + W 4096x7168 "
                               "(128x128) to E4M3 in one launch, block-scaled GEMM 4096x4096x7168 -> BF16",
                   "M": M, "N": N, "K": K, "scale_mode": "free"},
        "kernels": {
            "quantize_act_1x128": {"us": round(qa_us, 2), "GB/s": round(qa_gbs, 1),
                                   "frac_hbm": round(qa_gbs / HBM_PEAK_GBS, 4), "bytes": ACT_BYTES},
            "quantize_weight_128x128": {"us": round(qw_us, 2), "GB/s": round(qw_gbs, 1),
                                        "frac_hbm": round(qw_gbs / HBM_PEAK_GBS, 4), "bytes": WGT_BYTES},
            # both quantizers of the step in one launch (fp8q_quantize_linear)
            "quantize_linear_act_and_weight": {
                "us": round(ql_us, 2), "GB/s": round((ACT_BYTES + WGT_BYTES) / ql_us / 1e3, 1),
                "frac_hbm": round((ACT_BYTES + WGT_BYTES) / ql_us / 1e3 / HBM_PEAK_GBS, 4),
                "bytes": ACT_BYTES + WGT_BYTES},
            "gemm_block_scaled": {"us": round(gemm_us, 2), "TFLOP/s": round(gemm_tflops, 1),
                                  "frac_fp8_mfma": round(gemm_tflops / FP8_PEAK_TFLOPS, 4), "flop": GEMM_FLOP},
            # the same GEMM with its 128-element partials formed inside the
            # FP8 matrix core (acc=FP8Q_ACC_FP8_MFMA); not used by the step
            "gemm_block_scaled_fp8_mfma": {"us": round(gemm_f8_us, 2), "TFLOP/s": round(gemm_f8_tflops, 1),
                                           "frac_fp8_mfma": round(gemm_f8_tflops / FP8_PEAK_TFLOPS, 4),
                                           "flop": GEMM_FLOP},
            # power-of-two scales applied by the matrix core, no promotion
            # (acc=FP8Q_ACC_FP8_MFMA_SCALED, inputs quantized with pow2 scales)
            "gemm_block_scaled_fp8_mfma_scaled_pow2": {
                "us": round(gemm_f8s_us, 2), "TFLOP/s": round(GEMM_FLOP / gemm_f8s_us / 1e6, 1),
                "frac_fp8_mfma": round(GEMM_FLOP / gemm_f8s_us / 1e6 / FP8_PEAK_TFLOPS, 4), "flop": GEMM_FLOP},
        },
        # single launches after a cache flush (the operands come from HBM)
        "gemm_block_scaled_after_cache_flush": {"median_us": round(flush_med_us, 2), "min_us": round(flush_min_us, 2),
                                                "launches": 20, "flush": "1 GiB written before each launch"},
        "quantize_linear_after_cache_flush": {
            "median_us": round(qflush_med_us, 2), "min_us": round(qflush_min_us, 2),
            "frac_hbm_median": round((ACT_BYTES + WGT_BYTES) / qflush_med_us / 1e3 / HBM_PEAK_GBS, 4),
            "launches": 20, "flush": "1 GiB written before each launch"},
        "gemm_quantized_output": {
            "workload": "4096x4096x7168 GEMM whose BF16 result is quantized 1x128 along N in the epilogue",
            "fused_us": round(gemm_q_us, 2), "fused_TFLOP/s": round(GEMM_FLOP / gemm_q_us / 1e6, 1),
            "unfused_gemm_bf16_plus_quantize_us": round(unfused_us, 2),
            "hbm_bytes_saved_per_call": M * N * 2 * 2},
        "quantize_only": quant_only,
        "moe_grouped": moe,
        "wgrad": wg,
        "dgrad": dg,
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": GEMM_TRAFFIC_BYTES},
        "cpu_baseline": None,
    }
    out["rocm_smi_clocks_after_run"] = rocm_smi_clocks()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
