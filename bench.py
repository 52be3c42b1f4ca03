"""Bench of the fine-grained FP8 linear-layer hot path on one MI355X.

One step = one pass of the path over the dense expert up-projection
(A BF16 4096 x 7168 with 0.1% outliers x100, W BF16 4096 x 7168 ~N(0, 0.02)):
1x128 online max-abs quantization of A and 128x128 quantization of W (one
launch, fp8q_quantize_linear), then the block-scaled FP8 GEMM to BF16
C[4096, 4096] (fp8q_gemm) -- all in libfp8q.so.  Inputs are generated on the
host (seeded), copied to HBM once, and are resident before the timed region
starts.

Timing:
  * before the --warmup untimed steps, the step runs for PREWARM_MS more
    (untimed), so the timed region sees the GPU's steady clock whatever
    --warmup is;
  * the timed region is exactly --steps steps between two synchronizations;
    inside it, HIP events on the launch stream bracket every GEMM launch,
    which gives the GEMM's live average duration (the roofline's `achieved`);
  * every other kernel figure is the median of per-launch HIP event
    durations after a time-based warm-up of that kernel (>= WARM_MS), so it
    does not depend on what ran before it; quantizers rotate over copies of
    their inputs larger than the 256 MB Infinity Cache; `after_cache_flush`
    figures write 1 GiB before each launch.

Prints one JSON line (contract fields first; `workloads` holds every other
workload: tiny linear, Dgrad, quantize-only sizes, MoE grouped GEMMs and
glue, weight gradient; `cpu_baseline` times the oracle on the host and
checks a sample of the timed step's outputs against it).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]
"""

import argparse
import hashlib
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
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
METRIC = "block-scaled FP8 GEMM TFLOP/s + quantize GB/s, % of MI355X roofline"
PREWARM_MS = 300.0
WARM_MS = 100.0

# algorithmic bytes: BF16 read + code write + one float32 scale per tile
ACT_BYTES = M * K * 2 + M * K + M * (K // 128) * 4
WGT_BYTES = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
GEMM_FLOP = 2.0 * M * N * K
# codes and scales read once, BF16 C written once
GEMM_MIN_BYTES = M * K + N * K + M * (K // 128) * 4 + (N // 128) * (K // 128) * 4 + M * N * 2

# HBM traffic of one dense-GEMM launch from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE; each scaled by what the counter reads for a plain
# copy of known size), valid only for the kernel source it was measured on:
# when csrc/gemm.hip no longer hashes to `source_sha256` the bench reports
# traffic null.
GEMM_TRAFFIC = {"bytes": 216190000,
                "source_sha256": "5d0102877e6675f5b3e375937b8be0ce3ee28db1d42af65db226de7d529d2918",
                "profile": "profiles/bench_workloads_kernel_trace_and_hbm_traffic.md (FETCH_SIZE 88,416.8 KiB x 2.000 "
                           "+ WRITE_SIZE 34,307.4 KiB per launch of gemm_bs_kernel<0, 1, 0, 0>)"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (torch) --steps times; used to "
                        "scale the FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 --pmc run")
    return p.parse_args()


def source_sha256(name):
    with open(os.path.join(ROOT, "fine_grained_fp8_fp8q_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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


# ------------------------------------------------------------ timing ----

class Clock:
    """HIP-event timing on one stream."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self._scratch = None

    def _ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def warm(self, fn, ms=WARM_MS):
        """Launch fn(i) back to back for at least `ms` milliseconds."""
        t0 = time.perf_counter()
        i = 0
        while True:
            for _ in range(8):
                if fn(i) != 0:
                    raise RuntimeError("fp8q call failed")
                i += 1
            self.torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                return

    def launches(self, fn, reps, flush=False):
        """Per-launch durations (us) of fn(0..reps-1): back to back, one event
        between consecutive launches; with flush=True each launch follows a
        1 GiB write and has its own event pair."""
        if not flush:
            ev = [self._ev() for _ in range(reps + 1)]
            ev[0].record(self.stream)
            for i in range(reps):
                if fn(i) != 0:
                    raise RuntimeError("fp8q call failed")
                ev[i + 1].record(self.stream)
            ev[-1].synchronize()
            return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]
        if self._scratch is None:
            self._scratch = self.torch.empty(1 << 30, dtype=self.torch.uint8, device="cuda:0")
        out = []
        for i in range(reps):
            self._scratch.fill_(i & 0xFF)
            e0, e1 = self._ev(), self._ev()
            e0.record(self.stream)
            if fn(i) != 0:
                raise RuntimeError("fp8q call failed")
            e1.record(self.stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3)
        return out

    def batch(self, fn, reps):
        """Average duration (us) of fn(0..reps-1) launched back to back under
        one event pair: no event packet between the launches, so for a short
        kernel this is its own duration (a kernel trace shows consecutive
        launches of one stream starting as the previous one ends), where an
        event between every two launches adds its own processing to each."""
        e0, e1 = self._ev(), self._ev()
        e0.record(self.stream)
        for i in range(reps):
            if fn(i) != 0:
                raise RuntimeError("fp8q call failed")
        e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def stats(self, fn, reps, flop=None, nbytes=None, flush=False, warm=True):
        """Per-launch event median (and min) after a time-based warm-up; back
        to back, also the batch average of `reps` more launches under one event
        pair (`batch_avg_us`), from which the rates and fractions are taken."""
        if warm:
            self.warm(fn)
        t = self.launches(fn, reps, flush)
        med = float(np.median(t))
        r = {"median_us": round(med, 2), "min_us": round(float(np.min(t)), 2), "launches": reps}
        use = med
        if not flush:
            use = self.batch(fn, reps)
            r["batch_avg_us"] = round(use, 2)
        if flop is not None:
            r["TFLOP/s"] = round(flop / use / 1e6, 1)
            r["frac_fp8_peak"] = round(flop / use / 1e6 / FP8_PEAK_TFLOPS, 4)
        if nbytes is not None:
            r["GB/s"] = round(nbytes / use / 1e3, 1)
            r["frac_hbm"] = round(nbytes / use / 1e3 / HBM_PEAK_GBS, 4)
            r["bytes"] = int(nbytes)
        return r

    def after_idle(self, fn, reps=20):
        """Median of the first `reps` launches after 200 ms without GPU work
        (the HBM-bound kernels run faster in the first ~1.5 ms of load)."""
        self.torch.cuda.synchronize()
        time.sleep(0.2)
        return float(np.median(self.launches(fn, reps)))

    def release(self):
        self._scratch = None


def roofline_entry(flop, nbytes, med_us):
    """Time at the roofline max(flop / FP8 peak, bytes / HBM peak) and the
    fraction of it reached in med_us."""
    t = max(flop / (FP8_PEAK_TFLOPS * 1e6), nbytes / (HBM_PEAK_GBS * 1e3))
    return {"roofline_us": round(t, 2), "frac_roofline": round(t / med_us, 4),
            "bound": "mfma" if flop / (FP8_PEAK_TFLOPS * 1e6) >= nbytes / (HBM_PEAK_GBS * 1e3) else "hbm"}


# -------------------------------------------------------- workloads ----

def progress(msg):
    """One line on stderr as each part of the run completes (the JSON line
    alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def plain_stream(torch, clock, sp, n_elems, reps, rot):
    """The rate of a bare stream with a quantizer's traffic: the same number
    of elements through libfp8q_streamref.so's 2:1 kernel (2 B read, 1 B
    written per element, no arithmetic), over `rot` buffer sets like the
    quantizer it stands next to."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fine_grained_fp8_fp8q_amd", "libfp8q_streamref.so"))
    lib.fp8q_streamref_2to1.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.fp8q_streamref_2to1.restype = ctypes.c_int
    n = (n_elems + 15) // 16 * 16
    xs = [torch.empty(2 * n, dtype=torch.uint8, device="cuda:0") for _ in range(rot)]
    ys = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(rot)]
    r = clock.stats(lambda i: lib.fp8q_streamref_2to1(xs[i % rot].data_ptr(), ys[i % rot].data_ptr(), n, sp),
                    reps, nbytes=3 * n)
    return {"elements": n, "batch_avg_us": r["batch_avg_us"], "frac_hbm": r["frac_hbm"]}


def with_stream(r, ps):
    """Attach the same-size bare stream to a quantizer's entry."""
    r["plain_stream_same_elements"] = ps
    r["frac_of_plain_stream"] = round(ps["batch_avg_us"] / r["batch_avg_us"], 3)
    return r


def bf16_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def graph_replay_us(torch, fn, reps=20, min_ms=100.0, replays=50):
    """GPU time (us) per call of fn(stream), from a HIP graph holding `reps`
    calls, replayed back to back (after `min_ms` of untimed replays) under one
    event pair: without the host's cost of each call, which for a kernel of a
    few microseconds is longer than the kernel itself."""
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for _ in range(reps):
            if fn(gs.cuda_stream) != 0:
                raise RuntimeError("fp8q call failed during graph capture")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    e1.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / (reps * replays), 2), g


def tiny_linear(torch, fp8q, lib, clock, sp):
    """Tiny linear, 128 x 256 x 512, FP32 out: latency of one pass (quantize A and
    W in one launch, then the GEMM), and of each kernel.  Launched one call at a
    time from the host, a pass of a few microseconds is timed as the host's call
    rate; `graph_replay` gives the GPU's own time per pass (and per kernel) from
    HIP graphs of 20 passes, and checks that a replayed pass writes exactly what
    the eager pass wrote."""
    import synth
    d = synth.tiny_linear()
    a, w = bf16_dev(torch, d["a"]), bf16_dev(torch, d["w"])
    m, k = a.shape
    n = w.shape[0]
    ac, as_, wc, ws = fp8q.quantize_linear(a, w)
    c = torch.empty((m, n), dtype=torch.float32, device="cuda:0")

    def q_on(s):
        return lib.fp8q_quantize_linear(a.data_ptr(), m, k, k, fp8q.SCALE_FREE, ac.data_ptr(), ac.stride(0),
                                        as_.data_ptr(), w.data_ptr(), n, k, fp8q.SCALE_FREE, wc.data_ptr(),
                                        wc.stride(0), ws.data_ptr(), s)

    def g_on(s):
        return lib.fp8q_gemm(ac.data_ptr(), as_.data_ptr(), wc.data_ptr(), ws.data_ptr(), m, n, k, fp8q.OUT_F32,
                             c.data_ptr(), n, s)

    def step_on(s):
        return q_on(s) or g_on(s)

    res = {"workload": "tiny linear: quantize A 128x512 (1x128) + W 256x512 (128x128), GEMM -> FP32 [128, 256]",
           "step_latency": clock.stats(lambda i: step_on(sp), 200),
           "quantize_linear": clock.stats(lambda i: q_on(sp), 200),
           "gemm": clock.stats(lambda i: g_on(sp), 200, flop=2.0 * m * n * k)}
    # the eager pass's output, then the same pass replayed from a graph
    if step_on(sp) != 0:
        raise RuntimeError("fp8q call failed")
    torch.cuda.synchronize()
    want = (ac.clone(), as_.clone(), wc.clone(), ws.clone(), c.clone())
    for t in (ac, as_, wc, ws, c):
        t.zero_()
    step_us, graph = graph_replay_us(torch, step_on)
    got = (ac, as_, wc, ws, c)
    same = all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(got, want))
    del graph
    q_us, _ = graph_replay_us(torch, q_on)
    g_us, _ = graph_replay_us(torch, g_on)
    res["graph_replay"] = {"step_us": step_us, "quantize_linear_us": q_us, "gemm_us": g_us,
                           "gemm_TFLOP/s": round(2.0 * m * n * k / g_us / 1e6, 1),
                           "passes_per_graph": 20, "replays_timed": 50,
                           "replayed_outputs_identical_to_eager": bool(same)}
    return res


def quantize_only(torch, fp8q, lib, clock, sp, reps):
    """Quantize-only sizes: activations 16384 x 7168 (Student-t(3)) in both scale modes,
    weights 7168 x 18432 per 128 x 128 block; two input/output sets, each
    larger than the Infinity Cache, alternate."""
    import synth
    out = {}
    act = synth.quant_only_act()
    rows, cols = act.shape
    xs = [bf16_dev(torch, act)]
    xs.append(xs[0].clone())
    cs = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    ss = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda:0")
    abytes = rows * cols * 3 + rows * (cols // 128) * 4
    for mode_name, mode in (("free", fp8q.SCALE_FREE), ("pow2", fp8q.SCALE_POW2)):
        def fn(i, mode=mode):
            return lib.fp8q_quantize_act(xs[i & 1].data_ptr(), rows, cols, cols, fp8q.TILE_ROW, mode,
                                         cs[i & 1].data_ptr(), cols, ss.data_ptr(), sp)
        r = clock.stats(fn, reps, nbytes=abytes)
        r["median_us_first_20_after_idle"] = round(clock.after_idle(fn), 2)
        out[f"act_16384x7168_{mode_name}"] = r
    del xs, cs, ss
    ps = plain_stream(torch, clock, sp, rows * cols, reps, 2)
    for mode_name in ("free", "pow2"):
        with_stream(out[f"act_16384x7168_{mode_name}"], ps)
    wt = synth.quant_only_weight()
    n, k = wt.shape
    ws = [bf16_dev(torch, wt)]
    ws.append(ws[0].clone())
    cs = [torch.empty((n, k), dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    ss = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda:0")
    wbytes = n * k * 3 + (n // 128) * (k // 128) * 4

    def fw(i):
        return lib.fp8q_quantize_weight(ws[i & 1].data_ptr(), n, k, k, fp8q.SCALE_FREE, cs[i & 1].data_ptr(), k,
                                        ss.data_ptr(), sp)
    r = clock.stats(fw, reps, nbytes=wbytes)
    r["median_us_first_20_after_idle"] = round(clock.after_idle(fw), 2)
    out["weight_7168x18432"] = r
    del ws, cs, ss
    with_stream(r, plain_stream(torch, clock, sp, n * k, reps, 2))
    return out


def moe(torch, fp8q, lib, clock, sp, reps):
    """MoE grouped GEMMs, one GPU's share of the MoE layer: 8192 tokens routed top-8
    over 256 experts (Zipf(1.1) popularity), 16 hosted experts (one empty).
    Tokens are quantized once (1x128), their codes and scales gathered by
    expert (FP8 dispatch gather); grouped up-projection 7168 -> 4096 and
    down-projection 2048 -> 7168, BF16 out; SwiGLU fused with the 1x128
    quantization of its output; the whole expert FFN forward as one pass."""
    import synth
    d = synth.moe_grouped()
    G = len(d["counts"])
    rows = int(d["counts"].sum())
    k_up = d["x"].shape[1]
    x = bf16_dev(torch, d["x"])
    xq, xs = fp8q.quantize_act(x)
    gather = torch.from_numpy(d["gather"].astype(np.int32)).to("cuda:0")
    a_up, s_up = fp8q.gather_rows(xq, xs, gather)
    off = torch.from_numpy(d["offsets"]).to("cuda:0")
    hq, hs = fp8q.quantize_act(bf16_dev(torch, d["h"]))
    # power-of-two operands for the fp32_pow2 form
    xq2, xs2 = fp8q.quantize_act(x, scale_mode="pow2")
    a_up2, s_up2 = fp8q.gather_rows(xq2, xs2, gather)
    hq2, hs2 = fp8q.quantize_act(bf16_dev(torch, d["h"]), scale_mode="pow2")
    del xq2, xs2
    out = {"experts": G, "rows_per_expert": [int(v) for v in d["counts"]], "rows": rows}

    nb_up = k_up // 128
    srcs = [(xq, xs)] + [fp8q.quantize_act(x) for _ in range(4)]  # > Infinity Cache in rotation

    def fg(i):
        q, sc = srcs[i % len(srcs)]
        return lib.fp8q_gather_rows(q.data_ptr(), q.shape[0], k_up, q.stride(0), sc.data_ptr(), gather.data_ptr(),
                                    rows, a_up.data_ptr(), a_up.stride(0), s_up.data_ptr(), sp)
    gbytes = 2 * rows * (k_up + nb_up * 4) + rows * 4
    out["dispatch_gather_fp8"] = clock.stats(fg, reps, nbytes=gbytes)

    inter = d["w_down"].shape[2]
    sx0 = bf16_dev(torch, synth.swiglu_input(rows=rows, inter=inter))
    sxs = [sx0] + [sx0.clone() for _ in range(9)]
    sq = torch.empty((rows, inter), dtype=torch.uint8, device="cuda:0")
    ssc = torch.empty((rows, inter // 128), dtype=torch.float32, device="cuda:0")
    cq = torch.empty((rows, 2 * inter), dtype=torch.uint8, device="cuda:0")
    cs = torch.empty((rows, 2 * inter // 128), dtype=torch.float32, device="cuda:0")
    for name, cache in (("swiglu_quantize", False), ("swiglu_quantize_with_pow2_cache", True)):
        def fs(i, cache=cache):
            return lib.fp8q_swiglu_quantize(sxs[i % len(sxs)].data_ptr(), rows, inter, 2 * inter, fp8q.SCALE_FREE,
                                            sq.data_ptr(), inter, ssc.data_ptr(), fp8q.SCALE_POW2,
                                            cq.data_ptr() if cache else None, 2 * inter,
                                            cs.data_ptr() if cache else None, sp)
        sbytes = rows * 2 * inter * 2 + rows * inter + rows * (inter // 128) * 4
        if cache:
            sbytes += rows * 2 * inter + rows * (2 * inter // 128) * 4
        out[name] = clock.stats(fs, reps, nbytes=sbytes)
        # a bare 2:1 stream moving the same number of bytes (the kernel's mix
        # is 4:1 reads to writes): the rate a plain stream of this size gets
        ps = plain_stream(torch, clock, sp, sbytes // 3, reps, 2)
        out[name]["plain_stream_same_bytes"] = ps
        out[name]["frac_of_plain_stream"] = round(ps["batch_avg_us"] / out[name]["batch_avg_us"], 3)
    del sxs, sx0, cq, cs

    weights = {}
    for name, wname, in_a, in_s, in_a2, in_s2 in (("up_7168x4096", "w_up", a_up, s_up, a_up2, s_up2),
                                                  ("down_2048x7168", "w_down", hq, hs, hq2, hs2)):
        wb = bf16_dev(torch, d[wname])
        g, n, k = wb.shape
        wq, wsc = fp8q.quantize_weight(wb.view(g * n, k))
        wq2, wsc2 = fp8q.quantize_weight(wb.view(g * n, k), scale_mode="pow2")
        del wb
        weights[wname] = (wq, wsc, n, k)
        c = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda:0")
        flop = 2.0 * rows * n * k
        nbytes = G * n * k + (G * n // 128) * (k // 128) * 4 + rows * k + rows * (k // 128) * 4 + rows * n * 2
        per = 0.0  # sum of each expert's own roofline time
        for m in d["counts"]:
            if m:
                per += max(2.0 * int(m) * n * k / (FP8_PEAK_TFLOPS * 1e6),
                           (n * k + (n // 128) * (k // 128) * 4 + int(m) * (k + (k // 128) * 4 + n * 2))
                           / (HBM_PEAK_GBS * 1e3))
        for acc_name, acc in (("", fp8q.ACC_FP32), ("_fp8_mfma", fp8q.ACC_FP8_MFMA),
                              ("_fp32_pow2", fp8q.ACC_FP32_POW2)):
            p2 = acc == fp8q.ACC_FP32_POW2
            ops = (in_a2, in_s2, wq2, wsc2) if p2 else (in_a, in_s, wq, wsc)

            def fn(i, acc=acc, ops=ops, n=n, k=k, c=c):
                return lib.fp8q_grouped_gemm_ex(ops[0].data_ptr(), ops[1].data_ptr(), off.data_ptr(), G, rows,
                                                ops[2].data_ptr(), ops[3].data_ptr(), n, k, fp8q.OUT_BF16, acc,
                                                c.data_ptr(), n, sp)
            r = clock.stats(fn, reps, flop=flop, nbytes=nbytes)
            r.update(roofline_entry(flop, nbytes, r.get("batch_avg_us", r["median_us"])))
            r["per_expert_roofline_us"] = round(per, 2)
            out[name + acc_name] = r
        del c, wq2, wsc2

    wq_u, ws_u, n_u, k_u = weights["w_up"]
    wq_d, ws_d, n_d, k_d = weights["w_down"]
    up_out = torch.empty((rows, n_u), dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty((rows, n_d), dtype=torch.bfloat16, device="cuda:0")

    def ffn(i):
        st = fg(i)
        st = st or lib.fp8q_grouped_gemm(a_up.data_ptr(), s_up.data_ptr(), off.data_ptr(), G, rows, wq_u.data_ptr(),
                                         ws_u.data_ptr(), n_u, k_u, fp8q.OUT_BF16, up_out.data_ptr(), n_u, sp)
        st = st or lib.fp8q_swiglu_quantize(up_out.data_ptr(), rows, inter, n_u, fp8q.SCALE_FREE, sq.data_ptr(),
                                            inter, ssc.data_ptr(), fp8q.SCALE_POW2, None, 0, None, sp)
        st = st or lib.fp8q_grouped_gemm(sq.data_ptr(), ssc.data_ptr(), off.data_ptr(), G, rows, wq_d.data_ptr(),
                                         ws_d.data_ptr(), n_d, k_d, fp8q.OUT_BF16, y.data_ptr(), n_d, sp)
        return st
    flop = 2.0 * rows * (n_u * k_u + n_d * k_d)
    r = clock.stats(ffn, reps, flop=flop)
    r["steps"] = "dispatch gather, grouped up GEMM, SwiGLU + quantize, grouped down GEMM"
    out["expert_ffn_forward"] = r
    return out


def wgrad(torch, fp8q, lib, clock, sp, reps, sample=None):
    """Weight gradient: dY 16384 x 2048 and X 16384 x 7168 (BF16 ~N(0,1)) quantized
    in 128-token x 1-feature tiles (codes feature-major), then
    dW[2048, 7168] = dY^T X in FP32.

    With `sample` = (dW rows, dW columns), also returns what the GPU computed
    there for the promotion study: dW of every accumulation form and the
    sampled features' codes and scales (free and power-of-two)."""
    import synth
    d = synth.wgrad()
    out = {}
    q = {}
    study = None
    if sample is not None:
        rs, cs = (torch.as_tensor(v, device="cuda:0") for v in sample)
        study = {"dw": {}, "operands": {}}
    for name, arr in (("dy", d["dy"]), ("x", d["x"])):
        t = bf16_dev(torch, arr)
        tok, feat = t.shape
        codes = torch.empty((feat, tok), dtype=torch.uint8, device="cuda:0")
        scales = torch.empty((feat, tok // 128), dtype=torch.float32, device="cuda:0")
        t2 = t.clone()

        def fn(i, ts=(t, t2), tok=tok, feat=feat, codes=codes, scales=scales):
            return lib.fp8q_quantize_act(ts[i & 1].data_ptr(), tok, feat, feat, fp8q.TILE_TOKEN_T, fp8q.SCALE_FREE,
                                         codes.data_ptr(), tok, scales.data_ptr(), sp)
        nbytes = tok * feat * 3 + feat * (tok // 128) * 4
        out[f"quantize_{name}_token_t_{tok}x{feat}"] = with_stream(
            clock.stats(fn, reps, nbytes=nbytes), plain_stream(torch, clock, sp, tok * feat, reps, 2))
        fn(0)
        q[name] = (codes, scales, tok, feat) + fp8q.quantize_act(t, tile_axis="token_t", scale_mode="pow2")
        del t, t2
    dyc, dys, T, nout, dyc2, dys2 = q["dy"]
    xc, xs, _, kin, xc2, xs2 = q["x"]
    if study is not None:
        for mode, ops in (("free", (dyc, dys, xc, xs)), ("pow2", (dyc2, dys2, xc2, xs2))):
            study["operands"][mode] = {k: v.cpu().numpy() for k, v in zip(
                ("dyc", "dys", "xc", "xs"), (ops[0][rs], ops[1][rs], ops[2][cs], ops[3][cs]))}
    dw = torch.empty((nout, kin), dtype=torch.float32, device="cuda:0")
    flop = 2.0 * nout * kin * T
    nbytes = (nout + kin) * T + (nout + kin) * (T // 128) * 4 + nout * kin * 4
    for acc_name, acc in (("", fp8q.ACC_FP32), ("_fp8_mfma", fp8q.ACC_FP8_MFMA), ("_fp32_pow2", fp8q.ACC_FP32_POW2),
                          ("_fp8_mfma_scaled_pow2", fp8q.ACC_FP8_MFMA_SCALED)):
        p2 = acc in (fp8q.ACC_FP32_POW2, fp8q.ACC_FP8_MFMA_SCALED)
        ops = (dyc2, dys2, xc2, xs2) if p2 else (dyc, dys, xc, xs)

        def fg(i, acc=acc, ops=ops):
            return lib.fp8q_wgrad_ex(ops[0].data_ptr(), ops[1].data_ptr(), ops[2].data_ptr(), ops[3].data_ptr(), nout,
                                     kin, T, acc, dw.data_ptr(), kin, sp)
        r = clock.stats(fg, reps, flop=flop, nbytes=nbytes)
        r.update(roofline_entry(flop, nbytes, r.get("batch_avg_us", r["median_us"])))
        out[f"wgrad_{nout}x{kin}x{T}{acc_name}"] = r
        if study is not None:
            assert fg(0) == 0
            study["dw"][acc_name] = dw[rs][:, cs].cpu().numpy().astype(np.float64)
    return out, study


def dgrad(torch, fp8q, lib, clock, sp, reps, w):
    """Activation gradient of the up-projection: W [4096, 7168] quantized once
    into both orientations, then dX [4096, 7168] = dY [4096, 4096] . W
    (reduction over N = 4096), dY BF16 ~N(0,1) in 1x128 tiles along N."""
    import synth
    n, k = w.shape
    m = 4096
    codes = torch.empty((n, k), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda:0")
    codes_t = torch.empty((k, n), dtype=torch.uint8, device="cuda:0")
    scales_t = torch.empty((k // 128, n // 128), dtype=torch.float32, device="cuda:0")
    w2 = [w, w.clone()]

    def fq(i):
        return lib.fp8q_quantize_weight_t(w2[i & 1].data_ptr(), n, k, k, fp8q.SCALE_FREE, codes.data_ptr(), k,
                                          scales.data_ptr(), codes_t.data_ptr(), n, scales_t.data_ptr(), sp)
    qbytes = n * k * 4 + 2 * (n // 128) * (k // 128) * 4
    out = {"quantize_weight_both_orientations_4096x7168": clock.stats(fq, reps, nbytes=qbytes)}
    rng = np.random.default_rng(21)
    dy = bf16_dev(torch, synth.bf16_rne(rng.standard_normal((m, n)).astype(np.float32)))
    dyq, dys = fp8q.quantize_act(dy)
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda:0")
    flop = 2.0 * m * n * k
    nbytes = m * n + n * k + m * (n // 128) * 4 + (k // 128) * (n // 128) * 4 + m * k * 2
    # the same operands with power-of-two scales, for the fp32_pow2 form
    dyq2, dys2 = fp8q.quantize_act(dy, scale_mode="pow2")
    _, _, ct2, st2 = fp8q.quantize_weight_t(w, scale_mode="pow2", both=False)
    ct2 = ct2.contiguous()
    for acc_name, acc in (("", fp8q.ACC_FP32), ("_fp8_mfma", fp8q.ACC_FP8_MFMA), ("_fp32_pow2", fp8q.ACC_FP32_POW2),
                          ("_fp8_mfma_scaled_pow2", fp8q.ACC_FP8_MFMA_SCALED)):
        p2 = acc in (fp8q.ACC_FP32_POW2, fp8q.ACC_FP8_MFMA_SCALED)
        ops = (dyq2, dys2, ct2, st2) if p2 else (dyq, dys, codes_t, scales_t)

        def fg(i, acc=acc, ops=ops):
            return lib.fp8q_gemm_ex(ops[0].data_ptr(), ops[1].data_ptr(), ops[2].data_ptr(), ops[3].data_ptr(), m, k,
                                    n, fp8q.OUT_BF16, acc, dx.data_ptr(), k, sp)
        r = clock.stats(fg, reps, flop=flop, nbytes=nbytes)
        r.update(roofline_entry(flop, nbytes, r.get("batch_avg_us", r["median_us"])))
        out[f"dgrad_{m}x{k}x{n}{acc_name}"] = r
    return out


# ------------------------------------------------------ CPU baseline ----

def cpu_baseline(step_outputs):
    """The oracle, as it stands, on the host cores, on bounded samples of
    each workload (quantize and GEMM timed apart), and a parity check of
    a sample of the timed step's outputs against it.

    `value` is the oracle's block-scaled GEMM rate on the dense up-projection
    sample (the headline metric's GEMM)."""
    import threadpoolctl

    import synth
    from oracle import gemm as G, quantize as Q

    cores = len(os.sched_getaffinity(0))
    res = {}
    with threadpoolctl.threadpool_limits(cores):
        def timed(f):
            t0 = time.perf_counter()
            v = f()
            return v, time.perf_counter() - t0

        # 1: the whole tiny linear
        d = synth.tiny_linear()
        (qa, tqa) = timed(lambda: Q.quantize_rows(d["a"]))
        (qw, tqw) = timed(lambda: Q.quantize_blocks(d["w"]))
        (_, tg) = timed(lambda: G.gemm(qa[0], qa[1], qw[0], qw[1]))
        b1 = d["a"].size * 3.03125 + d["w"].size * 3.0
        res["tiny_linear_128x256x512"] = {"quantize_s": round(tqa + tqw, 4), "quantize_GB/s": round(b1 / (tqa + tqw) / 1e9, 4),
                                "gemm_s": round(tg, 4), "gemm_TFLOP/s": round(2.0 * 128 * 256 * 512 / tg / 1e12, 6),
                                "sample": "whole workload (A 128x512, W 256x512, C 128x256)"}
        # 2: dense up-projection, 2048 rows of A and of W
        d = synth.dense_up()
        rows = 2048
        a, w = np.ascontiguousarray(d["a"][:rows]), np.ascontiguousarray(d["w"][:rows])
        (qa, tqa) = timed(lambda: Q.quantize_rows(a))
        (qw, tqw) = timed(lambda: Q.quantize_blocks(w))
        (_, tg) = timed(lambda: G.gemm(qa[0], qa[1], qw[0], qw[1]))
        gemm2 = 2.0 * rows * rows * K / tg / 1e12
        b2 = a.size * 3.03125 + w.size * 3.0
        res["dense_up_4096x4096x7168"] = {"quantize_s": round(tqa + tqw, 3), "quantize_GB/s": round(b2 / (tqa + tqw) / 1e9, 4),
                             "gemm_s": round(tg, 3), "gemm_TFLOP/s": round(gemm2, 5),
                             "sample": f"A rows 0..{rows - 1}, W rows 0..{rows - 1}: GEMM {rows}x{rows}x{K}"}
        # 3: quantize-only, 4096 activation rows per mode and 2048 weight rows
        act = synth.quant_only_act()[:4096]
        (_, tf) = timed(lambda: Q.quantize_rows(act, Q.FREE))
        (_, tp) = timed(lambda: Q.quantize_rows(act, Q.POW2))
        wt = synth.quant_only_weight()[:2048]
        (_, tw) = timed(lambda: Q.quantize_blocks(wt))
        res["quantize_only"] = {"act_free_GB/s": round(act.size * 3.03125 / tf / 1e9, 4),
                                  "act_pow2_GB/s": round(act.size * 3.03125 / tp / 1e9, 4),
                                  "weight_GB/s": round(wt.size * 3.0 / tw / 1e9, 4),
                                  "seconds": round(tf + tp + tw, 3),
                                  "sample": "activation rows 0..4095 (both modes), weight rows 0..2047"}
        # 4: MoE: the busiest hosted expert's first 1024 rows, up-projection
        md = synth.moe_grouped()
        e = int(np.argmax(md["counts"]))
        lo = int(md["offsets"][e])
        xr = md["x"][md["gather"][lo:lo + 1024]]
        (qx, tq) = timed(lambda: Q.quantize_rows(xr))
        (qwe, tqw) = timed(lambda: Q.quantize_blocks(md["w_up"][e][:2048]))
        (_, tg) = timed(lambda: G.gemm(qx[0], qx[1], qwe[0], qwe[1]))
        res["moe_grouped_16_experts"] = {"quantize_s": round(tq + tqw, 3), "gemm_s": round(tg, 3),
                                "gemm_TFLOP/s": round(2.0 * xr.shape[0] * 2048 * xr.shape[1] / tg / 1e12, 5),
                                "sample": f"expert {e}: {xr.shape[0]} of its rows x 2048 of its 4096 up-projection columns"}
        del md
        # 5: Wgrad: 256 dY features x 1024 X features over all 16384 tokens
        wd = synth.wgrad()
        (qdy, tq1) = timed(lambda: Q.quantize_token_t(np.ascontiguousarray(wd["dy"][:, :256])))
        (qx5, tq2) = timed(lambda: Q.quantize_token_t(np.ascontiguousarray(wd["x"][:, :1024])))
        (_, tg) = timed(lambda: G.wgrad(qdy[0], qdy[1], qx5[0], qx5[1]))
        t_tok = wd["dy"].shape[0]
        res["wgrad_2048x7168x16384"] = {"quantize_s": round(tq1 + tq2, 3),
                          "quantize_GB/s": round(t_tok * 1280 * 3.03125 / (tq1 + tq2) / 1e9, 4),
                          "gemm_s": round(tg, 3), "gemm_TFLOP/s": round(2.0 * 256 * 1024 * t_tok / tg / 1e12, 5),
                          "sample": f"dW[0:256, 0:1024] over {t_tok} tokens"}
        del wd
        parity = step_parity(step_outputs, synth, Q, G)
    total = sum(v.get("seconds", v.get("quantize_s", 0) + v.get("gemm_s", 0)) for v in res.values())
    blas = [i.get("num_threads") for i in threadpoolctl.threadpool_info()]
    return {"value": res["dense_up_4096x4096x7168"]["gemm_TFLOP/s"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "the oracle's block-scaled GEMM on 2048 rows of A and W of the 4096x4096x7168 workload "
                      f"(value); every workload's sample timed apart in per_workload ({total:.1f} s in all)",
            "blas_threads": blas, "per_workload": res, "parity_on_timed_outputs": parity}


def promotion_emulators():
    """Promotion-interval study, CPU part (run before the GPU is opened: its
    worker processes are forks of this one).  On the seeded 65,536-element
    sample of dW of the weight-gradient workload (256 rows x 256 columns),
    the oracle's quantization and exact values (free and power-of-two
    scales) and its accumulation emulators on the free-scale operands: a
    float32 accumulator and 13/14/16/20-bit fixed-point ones, each promoted
    to float32 every 128 products and not at all."""
    import synth
    from oracle import quantize as Q
    from tests import promotion_sample as P

    t0 = time.perf_counter()
    d = synth.wgrad()
    t = d["dy"].shape[0]
    ops = {"free": P.operands(d, Q.FREE), "pow2": P.operands(d, Q.POW2)}
    del d
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    configs = P.emulator_configs(t)
    sums = P.emulate(ops["free"], configs, workers)
    emulated = {name: P.stats(sums[name], ops["free"]["exact"], ops["free"]["s"]) for name, _, _ in configs}
    return {"ops": ops, "emulated": emulated, "seconds": round(time.perf_counter() - t0, 1), "workers": workers}


def promotion_report(cpu, gpu):
    """The promotion study: the GPU's accumulation forms on the weight-
    gradient workload against the exact dW on the sample, next to the
    emulators (promotion every 128 elements: jp-study.kr doc 258368, 3rd
    paragraph)."""
    from tests import promotion_sample as P

    same = all(np.array_equal(np.asarray(gpu["operands"][m][k]).view(np.uint8),
                              np.asarray(cpu["ops"][m][k]).view(np.uint8))
               for m in ("free", "pow2") for k in ("dyc", "dys", "xc", "xs"))
    forms = {"interval_128_fp32_grade": ("free", ""), "interval_128_fp8_unit": ("free", "_fp8_mfma"),
             "pow2_no_promotion_fp32_grade": ("pow2", "_fp32_pow2"),
             "pow2_no_promotion_fp8_unit_hardware_scales": ("pow2", "_fp8_mfma_scaled_pow2")}
    return {"workload": "dW 2048x7168 over 16384 tokens (128-token tiles)",
            "sample": f"{P.SIDE} dW rows x {P.SIDE} columns = {P.SIDE * P.SIDE} elements (seed 2024)",
            "errors": "max and mean of |value - exact| / sum|a b|, median of |value - exact| / |exact|, "
                      "fraction within 1e-5 sum|a b| + 1e-6",
            "gpu_codes_and_scales_equal_oracle_on_sample": bool(same),
            "gpu": {name: P.stats(gpu["dw"][key], cpu["ops"][mode]["exact"], cpu["ops"][mode]["s"])
                    for name, (mode, key) in forms.items()},
            "emulated": cpu["emulated"],
            "emulator_seconds": cpu["seconds"], "emulator_workers": cpu["workers"]}


def step_parity(outs, synth, Q, G):
    """A sample of the timed step's outputs against the oracle: 16 rows of A
    and two 128-row weight blocks, codes and scales bit for bit, and the
    4096 C elements they span within the BF16 tolerance rule."""
    a_codes, a_scales, w_codes, w_scales, c_bits = outs
    d = synth.dense_up()
    rng = np.random.default_rng(99)
    rows = np.sort(rng.choice(M, 16, replace=False))
    blocks = np.sort(rng.choice(N // 128, 2, replace=False))
    wrows = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in blocks])
    qa_c, qa_s = Q.quantize_rows(d["a"][rows])
    qw_c, qw_s = Q.quantize_blocks(d["w"][wrows])
    codes_ok = (np.array_equal(a_codes[rows], qa_c) and np.array_equal(a_scales[rows].view(np.uint32),
                                                                        qa_s.view(np.uint32))
                and np.array_equal(w_codes[wrows], qw_c)
                and np.array_equal(w_scales[blocks].view(np.uint32), qw_s.view(np.uint32)))
    ref, s = G.gemm(qa_c, qa_s, qw_c, qw_s)
    ok = G.accept_bf16(c_bits[np.ix_(rows, wrows)], ref, s)
    return {"codes_and_scales_bit_exact": bool(codes_ok), "gemm_within_tolerance": int(ok.sum()),
            "gemm_checked": int(ok.size),
            "sample": f"A rows {rows.tolist()}, W blocks {blocks.tolist()} (rows {blocks[0] * 128}..+127, "
                      f"{blocks[1] * 128}..+127)"}


def rocm_smi_clocks():
    """Current clocks reported by rocm-smi (read after the measurements), or
    None where it is not available.  rocm-smi is a Python script: it is run
    by this interpreter as a child process, not through its `env` shebang."""
    import shutil
    import subprocess
    try:
        smi = shutil.which("rocm-smi")
        if smi is None:
            return None
        target = os.path.realpath(smi)
        cmd = [sys.executable, target] if target.endswith(".py") else [smi]
        r = subprocess.run(cmd + ["--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        cards = json.loads(r.stdout[r.stdout.index("{"):])
        card = cards[sorted(cards)[0]]
        return {k.strip(" :"): v for k, v in card.items()}
    except Exception:
        return None


# --------------------------------------------------------------- main ----

def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "fp8q runs on one GPU only: it has no multi-GPU path (no sharding, no "
                                   "collectives); run with --gpus 1"}))
        sys.exit(2)

    # the promotion study's CPU part forks worker processes: before torch
    # opens the GPU
    study_cpu = None if args.no_cpu_baseline else promotion_emulators()
    if study_cpu is not None:
        progress(f"promotion-study emulators done ({study_cpu['seconds']} s)")

    import torch
    import fine_grained_fp8_fp8q_amd as fp8q
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    lib = fp8q.load_library()
    dev = torch.device("cuda:0")
    d = synth.dense_up(m=M, n=N, k=K)
    a = bf16_dev(torch, d["a"])
    w = bf16_dev(torch, d["w"])
    a_codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    w_codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    a_scales = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    w_scales = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    clock = Clock(torch, stream)

    def gemm(i=0):
        return lib.fp8q_gemm(a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(), w_scales.data_ptr(), M, N,
                             K, fp8q.OUT_BF16, c.data_ptr(), N, sp)

    def q_both(i=0):
        return lib.fp8q_quantize_linear(a.data_ptr(), M, K, K, fp8q.SCALE_FREE, a_codes.data_ptr(), K,
                                        a_scales.data_ptr(), w.data_ptr(), N, K, fp8q.SCALE_FREE,
                                        w_codes.data_ptr(), K, w_scales.data_ptr(), sp)

    def step(i=0):
        st = q_both() or gemm()
        if st != fp8q.OK:
            raise RuntimeError(f"fp8q call failed with status {st}")
        return st

    clock.warm(step, PREWARM_MS)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly --steps steps; events on the launch stream
    # bracket each GEMM launch (the GEMM's live duration)
    g0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    g1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        if q_both() != fp8q.OK:
            raise RuntimeError("fp8q_quantize_linear failed")
        g0[i].record(stream)
        if gemm() != fp8q.OK:
            raise RuntimeError("fp8q_gemm failed")
        g1[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_events = ev0.elapsed_time(ev1) / args.steps
    gemm_live_us = float(np.mean([g0[i].elapsed_time(g1[i]) * 1e3 for i in range(args.steps)]))
    step_outputs = (a_codes.cpu().numpy(), a_scales.cpu().numpy(), w_codes.cpu().numpy(), w_scales.cpu().numpy(),
                    c.view(torch.int16).cpu().numpy().view(np.uint16))

    reps = max(20, args.steps // 2)
    ROT = 5  # quantizer inputs rotate over 5 copies: more than the Infinity Cache
    a_rot = [a] + [a.clone() for _ in range(ROT - 1)]
    w_rot = [w] + [w.clone() for _ in range(ROT - 1)]
    ac_rot = [torch.empty_like(a_codes) for _ in range(ROT)]
    wc_rot = [torch.empty_like(w_codes) for _ in range(ROT)]

    def q_act_i(i):
        return lib.fp8q_quantize_act(a_rot[i % ROT].data_ptr(), M, K, K, fp8q.TILE_ROW, fp8q.SCALE_FREE,
                                     ac_rot[i % ROT].data_ptr(), K, a_scales.data_ptr(), sp)

    def q_wgt_i(i):
        return lib.fp8q_quantize_weight(w_rot[i % ROT].data_ptr(), N, K, K, fp8q.SCALE_FREE, wc_rot[i % ROT].data_ptr(),
                                        K, w_scales.data_ptr(), sp)

    def q_lin_i(i):
        return lib.fp8q_quantize_linear(a_rot[i % ROT].data_ptr(), M, K, K, fp8q.SCALE_FREE, ac_rot[i % ROT].data_ptr(),
                                        K, a_scales.data_ptr(), w_rot[i % ROT].data_ptr(), N, K, fp8q.SCALE_FREE,
                                        wc_rot[i % ROT].data_ptr(), K, w_scales.data_ptr(), sp)

    dense = {"quantize_act_1x128": clock.stats(q_act_i, reps, nbytes=ACT_BYTES),
             "quantize_weight_128x128": clock.stats(q_wgt_i, reps, nbytes=WGT_BYTES),
             "quantize_linear_act_and_weight": clock.stats(q_lin_i, reps, nbytes=ACT_BYTES + WGT_BYTES)}
    ps = plain_stream(torch, clock, sp, M * K, reps, ROT)
    with_stream(dense["quantize_act_1x128"], ps)
    with_stream(dense["quantize_weight_128x128"], ps)
    with_stream(dense["quantize_linear_act_and_weight"], plain_stream(torch, clock, sp, M * K + N * K, reps, ROT))
    dense["quantize_linear_after_cache_flush"] = clock.stats(lambda i: q_lin_i(0), 20, nbytes=ACT_BYTES + WGT_BYTES,
                                                             flush=True)
    del a_rot, w_rot, ac_rot, wc_rot
    q_both()  # the step's codes again, for the GEMMs below

    # GEMM forms; the quantized-output GEMM next to the GEMM + quantizer pair
    # it replaces, measured in alternating rounds so all three see one clock
    cq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    cqs = torch.empty((M, N // 128), dtype=torch.float32, device=dev)

    def fused(i):
        return lib.fp8q_gemm_quantized(a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(),
                                       w_scales.data_ptr(), M, N, K, fp8q.ACC_FP32, fp8q.SCALE_FREE, cq.data_ptr(), N,
                                       cqs.data_ptr(), sp)

    def unfused(i):
        return gemm() or lib.fp8q_quantize_act(c.data_ptr(), M, N, N, fp8q.TILE_ROW, fp8q.SCALE_FREE, cq.data_ptr(),
                                               N, cqs.data_ptr(), sp)
    rounds = {"gemm": [], "fused": [], "unfused": []}
    for _ in range(3):
        for name, fn in (("gemm", gemm), ("fused", fused), ("unfused", unfused)):
            clock.warm(fn, WARM_MS / 2)
            rounds[name] += clock.launches(fn, max(10, reps // 3))
    med = {k: float(np.median(v)) for k, v in rounds.items()}
    dense["gemm_block_scaled"] = {"median_us": round(med["gemm"], 2), "min_us": round(float(np.min(rounds["gemm"])), 2),
                                  "launches": len(rounds["gemm"]), "TFLOP/s": round(GEMM_FLOP / med["gemm"] / 1e6, 1),
                                  "frac_fp8_peak": round(GEMM_FLOP / med["gemm"] / 1e6 / FP8_PEAK_TFLOPS, 4),
                                  "frac_bf16_peak": round(GEMM_FLOP / med["gemm"] / 1e6 / BF16_PEAK_TFLOPS, 4)}
    dense["gemm_quantized_output"] = {
        "workload": "the 4096x4096x7168 GEMM whose BF16 result is quantized 1x128 along N in its epilogue, next to "
                    "the GEMM (BF16 out) followed by the 1x128 quantizer",
        "fused_median_us": round(med["fused"], 2), "unfused_pair_median_us": round(med["unfused"], 2),
        "gemm_alone_median_us": round(med["gemm"], 2),
        "ordered_gemm_le_fused_le_unfused": bool(med["gemm"] <= med["fused"] <= med["unfused"]),
        "hbm_bytes_saved_per_call": M * N * 2 * 2}
    flushed = clock.stats(gemm, 20, flop=GEMM_FLOP, flush=True)
    dense["gemm_block_scaled_after_cache_flush"] = flushed
    del cq, cqs
    dense["gemm_block_scaled_fp8_mfma"] = clock.stats(
        lambda i: lib.fp8q_gemm_ex(a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(), w_scales.data_ptr(),
                                   M, N, K, fp8q.OUT_BF16, fp8q.ACC_FP8_MFMA, c.data_ptr(), N, sp), reps, flop=GEMM_FLOP)
    ap_c, ap_s, wp_c, wp_s = fp8q.quantize_linear(a, w, act_scale_mode="pow2", weight_scale_mode="pow2")
    dense["gemm_block_scaled_fp8_mfma_scaled_pow2"] = clock.stats(
        lambda i: lib.fp8q_gemm_ex(ap_c.data_ptr(), ap_s.data_ptr(), wp_c.data_ptr(), wp_s.data_ptr(), M, N, K,
                                   fp8q.OUT_BF16, fp8q.ACC_FP8_MFMA_SCALED, c.data_ptr(), N, sp), reps, flop=GEMM_FLOP)
    # float32 grade with power-of-two scales applied while widening (no fold)
    dense["gemm_block_scaled_fp32_pow2"] = clock.stats(
        lambda i: lib.fp8q_gemm_ex(ap_c.data_ptr(), ap_s.data_ptr(), wp_c.data_ptr(), wp_s.data_ptr(), M, N, K,
                                   fp8q.OUT_BF16, fp8q.ACC_FP32_POW2, c.data_ptr(), N, sp), reps, flop=GEMM_FLOP)
    dense["gemm_block_scaled_fp32_pow2"]["frac_bf16_peak"] = round(
        GEMM_FLOP / dense["gemm_block_scaled_fp32_pow2"]["batch_avg_us"] / 1e6 / BF16_PEAK_TFLOPS, 4)
    del ap_c, ap_s, wp_c, wp_s
    clock.release()

    progress("dense up-projection (timed steps, quantizers, GEMM forms) done")
    workloads = {"tiny_linear_128x256x512": tiny_linear(torch, fp8q, lib, clock, sp), "dense_up_4096x4096x7168": dense}
    progress("tiny linear done")
    workloads["dgrad_4096x7168x4096"] = dgrad(torch, fp8q, lib, clock, sp, reps, w)
    progress("Dgrad done")
    workloads["quantize_only"] = quantize_only(torch, fp8q, lib, clock, sp, reps)
    progress("quantize-only sizes done")
    workloads["moe_grouped_16_experts"] = moe(torch, fp8q, lib, clock, sp, reps)
    progress("MoE grouped done")
    sample = None if study_cpu is None else (study_cpu["ops"]["free"]["rsel"], study_cpu["ops"]["free"]["csel"])
    workloads["wgrad_2048x7168x16384"], study_gpu = wgrad(torch, fp8q, lib, clock, sp, reps, sample)
    progress("Wgrad done")

    traffic = GEMM_TRAFFIC["bytes"] if GEMM_TRAFFIC["source_sha256"] == source_sha256("gemm.hip") else None
    achieved = GEMM_FLOP / gemm_live_us / 1e6
    value = GEMM_FLOP / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x e4m3 -> f32 (bf16 in/out)",
        "data": "synthetic (seeded): A ~N(0,1) with 0.1% entries x100, W ~N(0,0.02), BF16",
        "config": {"workload": "dense expert up-projection: quantize A 4096x7168 (1x128) + W 4096x7168 (128x128) "
                               "to E4M3 in one launch, block-scaled GEMM 4096x4096x7168 -> BF16",
                   "M": M, "N": N, "K": K, "scale_mode": "free"},
        "ms_per_step_stream_events": round(ms_step_events, 4),
        "prewarm_ms": PREWARM_MS,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "gemm_bs_kernel, dense, float32-grade partials (fp8q_gemm)",
                     "flop_per_launch": GEMM_FLOP, "algorithmic_bytes_per_launch": GEMM_MIN_BYTES,
                     "launch_us_in_timed_steps": round(gemm_live_us, 2),
                     "frac_bf16_matrix_core_peak": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "back_to_back_median_us": dense["gemm_block_scaled"]["median_us"],
                     "frac_back_to_back": dense["gemm_block_scaled"]["frac_fp8_peak"],
                     "after_cache_flush_median_us": flushed["median_us"],
                     "frac_after_cache_flush": flushed["frac_fp8_peak"],
                     "traffic_source": (GEMM_TRAFFIC["profile"] if traffic is not None else
                                        "null: the kernel source changed since the counters were taken")},
        "cpu_baseline": None,
        "workloads": workloads,
        "pages_context": {
            "accumulation_interval_elements": 128,
            "accumulation_interval_hardware": "H800 tensor cores, four WGMMAs (jp-study.kr doc 258368, 3rd paragraph)",
            "full_training_h800_gpu_hours": 2.788e6,
            "full_training_source": "why-be.co.kr wr_id=77087, 1st paragraph",
            "note": "context only: the pages report no kernel throughput for this path"},
    }
    out["rocm_smi_clocks_after_run"] = rocm_smi_clocks()
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(step_outputs)
        out["promotion_study"] = promotion_report(study_cpu, study_gpu)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
