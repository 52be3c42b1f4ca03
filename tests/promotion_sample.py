"""The sample of dW elements the promotion study reports on: 256 rows x 256
columns of dW (65,536 elements) of the weight-gradient workload, drawn with
a fixed seed, the oracle's quantization and exact values there, and the
accumulation emulators run over it.  Shared by the GPU part of the study
(measured accumulation forms), its CPU part (emulators) and the bench's
report, so all of them report on the same elements.  Test infrastructure:
it calls the oracle."""

import multiprocessing
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle import accum, gemm as G, quantize as Q

SIDE = 256


def sample(nout, kin, seed=2024):
    """Sorted row and column indices of dW (SIDE each)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(nout, SIDE, replace=False)), np.sort(rng.choice(kin, SIDE, replace=False))


def operands(d, mode=Q.FREE):
    """The oracle's token-axis codes and scales of the sampled dY and X
    features, the sample indices, and the exact dW and S on the sample
    ([SIDE, SIDE] each, row-major like the sample)."""
    t, nout = d["dy"].shape
    rsel, csel = sample(nout, d["x"].shape[1])
    dyc, dys = Q.quantize_token_t(d["dy"][:, rsel], mode)
    xc, xs = Q.quantize_token_t(d["x"][:, csel], mode)
    exact, s = G.wgrad(dyc, dys, xc, xs)
    return {"rsel": rsel, "csel": csel, "dyc": dyc, "dys": dys, "xc": xc, "xs": xs, "exact": exact, "s": s}


def stats(value, exact, s):
    """Errors of `value` against the exact values: relative to S = sum |a b|
    (the tolerance's normalisation), the median relative to |exact|, and the
    fraction within the stated tolerance."""
    value, exact, s = (np.asarray(v, np.float64).ravel() for v in (value, exact, s))
    err = np.abs(value - exact)
    rel = err / s
    nz = exact != 0
    return {"max_err_over_S": float(rel.max()), "mean_err_over_S": float(rel.mean()),
            "median_err_over_abs": float(np.median(err[nz] / np.abs(exact[nz]))),
            "within_tolerance": float((err <= G.tolerance(s)).mean())}



WIDTHS = (13, 14, 16, 20)

# set before the worker processes fork (they read them, copy-on-write)
_SHARED = {}


def emulator_configs(t, widths=WIDTHS):
    """(name, promotion interval, accumulator width or None for float32):
    every width promoted every 128 products and not at all."""
    configs = [("fp32_interval_128", 128, None), ("fp32_no_promotion", t, None)]
    for w in widths:
        configs += [(f"fixed{w}_interval_128", 128, w), (f"fixed{w}_no_promotion", t, w)]
    return configs


def _emulate_chunk(bounds):
    lo, hi = bounds
    a, b, configs = _SHARED["a"], _SHARED["b"], _SHARED["configs"]
    r, c = np.arange(lo, hi) // SIDE, np.arange(lo, hi) % SIDE
    # the products (a sa)(b sb) of each sampled pair, as
    # accum.dequantized_products forms them; one column per product index,
    # so each accumulation step reads contiguous memory
    terms = np.asfortranarray(a[r] * b[c])
    return lo, {name: accum.accumulate(terms, interval, width) for name, interval, width in configs}


def emulate(ops, configs, workers, chunk=8192):
    """Every emulator of `configs` (oracle.accum.accumulate) on every sampled
    element, row-major over the sample; returns name -> float64 [SIDE^2].

    The sampled dY and X rows are dequantized once; chunks of `chunk`
    elements run in `workers` processes forked from this one, so call it only
    from a process that has not opened a GPU."""
    _SHARED.update(a=accum.dequantize(ops["dyc"], ops["dys"]), b=accum.dequantize(ops["xc"], ops["xs"]),
                   configs=configs)
    n = SIDE * SIDE
    sums = {name: np.empty(n) for name, _, _ in configs}
    try:
        with ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("fork")) as pool:
            for lo, part in pool.map(_emulate_chunk, [(lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]):
                for name, v in part.items():
                    sums[name][lo:lo + v.size] = v
    finally:
        _SHARED.clear()
    return sums
