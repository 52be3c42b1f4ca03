"""Bench of the fine-grained FP8 linear-layer hot path on one MI355X.

One step = one pass of the path over the dense expert up-projection
(A BF16 4096 x 7168 with 0.1% outliers x100, W BF16 4096 x 7168 ~N(0, 0.02)):
1x128 online max-abs quantization of A, 128x128 quantization of W, and the
block-scaled FP8 GEMM to BF16 C[4096, 4096] -- all three in libfp8q.so.
Inputs are generated on the host (seeded), copied to HBM once, and are
resident before the timed region starts.

Prints one JSON line:
  value      = whole-step throughput, 2*M*N*K / step time (TFLOP/s)
  kernels    = per-kernel average durations from HIP events recorded on the
               launch stream around each kernel in every timed step, with GB/s
               or TFLOP/s and the fraction of the MI355X roofline
  roofline   = the dominant kernel (the GEMM) against the dense FP8 MFMA peak
  cpu_baseline = the oracle timed on the host on a bounded sample

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
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
# traffic measured with rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, KiB per
# dispatch, scaled by a copy-kernel calibration) for the current GEMM kernel;
# None until measured for this kernel version
GEMM_TRAFFIC_BYTES = None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
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

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = lib.fp8q_quantize_act(a.data_ptr(), M, K, K, fp8q.TILE_ROW, fp8q.SCALE_FREE,
                                   a_codes.data_ptr(), K, a_scales.data_ptr(), sp)
        if ev is not None:
            ev[1].record(stream)
        st |= lib.fp8q_quantize_weight(w.data_ptr(), N, K, K, fp8q.SCALE_FREE, w_codes.data_ptr(), K,
                                       w_scales.data_ptr(), sp)
        if ev is not None:
            ev[2].record(stream)
        st |= lib.fp8q_gemm(a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(), w_scales.data_ptr(),
                            M, N, K, fp8q.OUT_BF16, c.data_ptr(), N, sp)
        if ev is not None:
            ev[3].record(stream)
        if st != fp8q.OK:
            raise RuntimeError(f"fp8q call failed with status {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / args.steps
    dur = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in events])  # ms
    qa_us, qw_us, gemm_us = (dur.mean(axis=0) * 1e3).tolist()
    qa_gbs = ACT_BYTES / (qa_us * 1e-6) / 1e9
    qw_gbs = WGT_BYTES / (qw_us * 1e-6) / 1e9
    gemm_tflops = GEMM_FLOP / (gemm_us * 1e-6) / 1e12
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
        "dtype": "fp8-e4m3 x fp8-e4m3 -> f32 accumulate, bf16 in/out",
        "data": "synthetic (seeded): A ~N(0,1) with 0.1% entries x100, W ~N(0,0.02), BF16",
        "config": {"workload": "dense expert up-projection: quantize A 4096x7168 (1x128) + W 4096x7168 "
                               "(128x128) to E4M3, block-scaled GEMM 4096x4096x7168 -> BF16",
                   "M": M, "N": N, "K": K, "scale_mode": "free"},
        "kernels": {
            "quantize_act_1x128": {"us": round(qa_us, 2), "GB/s": round(qa_gbs, 1),
                                   "frac_hbm": round(qa_gbs / HBM_PEAK_GBS, 4), "bytes": ACT_BYTES},
            "quantize_weight_128x128": {"us": round(qw_us, 2), "GB/s": round(qw_gbs, 1),
                                        "frac_hbm": round(qw_gbs / HBM_PEAK_GBS, 4), "bytes": WGT_BYTES},
            "gemm_block_scaled": {"us": round(gemm_us, 2), "TFLOP/s": round(gemm_tflops, 1),
                                  "frac_fp8_mfma": round(gemm_tflops / FP8_PEAK_TFLOPS, 4), "flop": GEMM_FLOP},
        },
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": GEMM_TRAFFIC_BYTES},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
