"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no arithmetic of the method: it draws random numbers and
rounds them to BF16 (the inputs' storage type), and builds the MoE routing
that decides which token rows each hosted expert receives.  Both the oracle
side and the GPU side of every test and of the bench take their inputs from
here; nothing else is shared between them.

Recipes (seed 0; one child stream per tensor from
``np.random.SeedSequence(seed).spawn``, drawn in a fixed order):

* tiny linear:   A 128x512 ~N(0,1) with round(0.5% * numel) distinct entries
                 x50; W 256x512 ~N(0, 0.02)
* dense up-proj: A 4096x7168 ~N(0,1) with 0.1% entries x100; W 4096x7168
                 ~N(0, 0.02) (gate rows 0..2047, up rows 2048..4095)
* quantize-only: activations 16384x7168 standard Student-t(3); weights
                 7168x18432 ~N(0, 0.02)
* MoE grouped:   8192 tokens x 7168 ~N(0,1) with 0.1% x100; expert
                 popularity p ~ rank^-1.1 over a random ranking of 256
                 experts; each token takes 8 distinct experts by Gumbel-top-k
                 on log p; this GPU hosts experts 0..15 and the least popular
                 hosted expert is masked so one group is empty; up W
                 [16, 4096, 7168], down W [16, 7168, 2048] ~N(0, 0.02); the
                 down-projection input is [sum M, 2048] ~N(0,1)
* Wgrad:         dY 16384x2048 and X 16384x7168 ~N(0,1)
* SwiGLU input:  the up-projection output of the MoE workload's rows,
                 [sum M, 4096] (gate | up) ~N(0, 1.7): the spread of a sum
                 of 7168 N(0,1) x N(0, 0.02) products (sqrt(7168) * 0.02)

* codes/scales:  uniformly drawn finite E4M3 codes and positive float32
                 scales 2^U[-8, 8) * U[1, 2), for GEMM operands that are not
                 the quantization of a BF16 input

Outliers are multiplied in float32 before the BF16 rounding.  "N(0, 0.02)"
is read as standard deviation 0.02.
"""

import numpy as np

SEED = 0


def bf16_rne(x):
    """float32 array -> BF16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def streams(seed, count):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(count)]


def normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def add_outliers(rng, x, frac, factor):
    """Multiply round(frac * numel) distinct uniformly chosen entries by factor."""
    flat = x.reshape(-1)
    count = int(round(frac * flat.size))
    idx = rng.choice(flat.size, size=count, replace=False)
    flat[idx] *= np.float32(factor)
    return x


def tiny_linear(seed=SEED):
    r = streams(seed, 4)
    a = add_outliers(r[1], normal(r[0], (128, 512)), 0.005, 50.0)
    w = normal(r[2], (256, 512), 0.02)
    return {"a": bf16_rne(a), "w": bf16_rne(w)}


def dense_up(seed=SEED, m=4096, n=4096, k=7168):
    r = streams(seed, 4)
    a = add_outliers(r[1], normal(r[0], (m, k)), 0.001, 100.0)
    w = normal(r[2], (n, k), 0.02)
    return {"a": bf16_rne(a), "w": bf16_rne(w)}


def quant_only_act(seed=SEED, rows=16384, cols=7168):
    r = streams(seed, 4)
    x = r[0].standard_t(3, size=(rows, cols)).astype(np.float32)
    return bf16_rne(x)


def quant_only_weight(seed=SEED, n=7168, k=18432):
    r = streams(seed, 4)
    return bf16_rne(normal(r[1], (n, k), 0.02))


def moe_routing(seed=SEED, tokens=8192, experts=256, top_k=8, hosted=16, zipf=1.1):
    """Token lists of the hosted experts (Gumbel-top-k routing, one masked).

    Returns (token_idx list per hosted expert (ascending), counts array).
    """
    r = streams(seed, 8)
    rank = r[3].permutation(experts) + 1
    logp = -zipf * np.log(rank.astype(np.float64))
    g = r[4].gumbel(size=(tokens, experts))
    choice = np.argpartition(-(logp[None, :] + g), top_k - 1, axis=1)[:, :top_k]
    lists = []
    for e in range(hosted):
        lists.append(np.nonzero((choice == e).any(axis=1))[0].astype(np.int64))
    masked = int(np.argmax(rank[:hosted]))  # least popular hosted expert
    lists[masked] = np.zeros(0, dtype=np.int64)
    counts = np.array([len(v) for v in lists], dtype=np.int64)
    return lists, counts


def moe_grouped(seed=SEED, tokens=8192, hidden=7168, inter=2048, hosted=16,
                with_weights=True):
    """MoE grouped-GEMM inputs for one GPU's 16 hosted experts."""
    r = streams(seed, 8)
    x = bf16_rne(add_outliers(r[1], normal(r[0], (tokens, hidden)), 0.001, 100.0))
    lists, counts = moe_routing(seed, tokens=tokens, hosted=hosted)
    gather = np.concatenate(lists) if lists else np.zeros(0, dtype=np.int64)
    offsets = np.zeros(hosted + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    out = {"x": x, "gather": gather, "offsets": offsets, "counts": counts}
    total = int(counts.sum())
    out["h"] = bf16_rne(normal(r[5], (total, inter)))
    if with_weights:
        out["w_up"] = bf16_rne(normal(r[6], (hosted, 2 * inter, hidden), 0.02))
        out["w_down"] = bf16_rne(normal(r[7], (hosted, hidden, inter), 0.02))
    return out


def wgrad(seed=SEED, tokens=16384, nout=2048, kin=7168):
    r = streams(seed, 4)
    dy = bf16_rne(normal(r[0], (tokens, nout)))
    x = bf16_rne(normal(r[1], (tokens, kin)))
    return {"dy": dy, "x": x}


def swiglu_input(seed=SEED, rows=None, inter=2048):
    """BF16 [rows, 2*inter] (gate | up) ~N(0, 1.7); rows default to the MoE
    workload's hosted rows."""
    if rows is None:
        rows = int(moe_routing(seed)[1].sum())
    r = streams(seed + 1, 1)
    return bf16_rne(normal(r[0], (rows, 2 * inter), 1.7))


def reachable_band(ebits, seed):
    """Every (x, amax) pair with amax in one BF16 binade and |x| <= amax, as
    BF16 bit patterns [tiles, 128].

    Row i is a 128-element tile whose element 0 is the amax (random sign) and
    whose other elements are x values (random signs).  For each of the 128
    amax significands of binade `ebits` (BF16 exponent field), every BF16
    magnitude from 0 up to amax appears once.  A tile's scale and codes
    depend only on (x, amax) pairs, so the tiles of all 255 binades cover
    every input the 1x128 quantizer can see.
    """
    rng = np.random.default_rng(seed)
    tiles = []
    for mant in range(128):
        ab = (ebits << 7) | mant
        if ab == 0:
            continue
        xs = np.arange(0, ab + 1, dtype=np.uint32).astype(np.uint16)
        xs |= (rng.integers(0, 2, xs.size) << 15).astype(np.uint16)
        pad = (-xs.size) % 127
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        head = np.full((xs.shape[0], 1), ab, np.uint16) | (rng.integers(0, 2, (xs.shape[0], 1)) << 15).astype(np.uint16)
        tiles.append(np.concatenate([head, xs], axis=1))
    return np.concatenate(tiles)



def e4m3_codes(rng, shape):
    """Uniformly drawn E4M3 bit patterns over the finite codes: the two NaN
    patterns (0x7F, 0xFF) are replaced by the largest finite codes of the
    same sign (0x7E, 0xFE), since no quantizer emits a NaN."""
    n = int(np.prod(shape))
    c = np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()
    c[(c & 0x7F) == 0x7F] -= 1
    return c


def tile_scales(rng, shape):
    """Positive float32 scales 2^e * m, e uniform in [-8, 8), m uniform in
    [1, 2): free scales with full float32 mantissas."""
    e = rng.integers(-8, 8, size=shape)
    m = rng.uniform(1.0, 2.0, size=shape)
    return (np.ldexp(m, e)).astype(np.float32)
