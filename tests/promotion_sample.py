"""The sample of dW elements the promotion study reports on: 256 rows x 256
columns of dW (65,536 elements) of the weight-gradient workload, drawn with
a fixed seed, and the oracle's quantization and exact values there.  Shared
by the GPU part of the study (measured accumulation forms) and its CPU part
(accumulation emulators), so both report on the same elements."""

import numpy as np

from oracle import gemm as G, quantize as Q

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

