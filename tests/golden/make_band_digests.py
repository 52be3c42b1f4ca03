"""Writes tests/golden/reachable_band_digests.txt: for every BF16 exponent
field 0..254 and both scale modes, the SHA-256 of the oracle's 1x128
quantization (codes, then float32 scales, as little-endian bytes) of the
tiles synth.reachable_band(ebits, seed=ebits) -- every (x, amax) pair of
that binade.  Calls only oracle/ and synth/ (jp-study.kr doc 258368 ¶1:
online max-abs per 1x128 tile; tmdrlife.com wr_id=13334 ¶4: power-of-two
scales).

    python tests/golden/make_band_digests.py
"""

import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import quantize as Q  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "reachable_band_digests.txt")


def digest(codes, scales):
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(codes, dtype=np.uint8).tobytes())
    h.update(np.ascontiguousarray(scales, dtype="<f4").tobytes())
    return h.hexdigest()


def main():
    lines = ["# SHA-256 of oracle.quantize.quantize_rows(synth.reachable_band(e, seed=e), mode):",
             "# codes bytes then float32 scale bytes; written by tests/golden/make_band_digests.py",
             "# columns: exponent field, mode, tiles, digest"]
    for ebits in range(255):
        bits = synth.reachable_band(ebits, seed=ebits)
        for mode in (Q.FREE, Q.POW2):
            codes, scales = Q.quantize_rows(bits, mode)
            lines.append(f"{ebits} {mode} {bits.shape[0]} {digest(codes, scales)}")
        print(ebits, bits.shape[0], flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
