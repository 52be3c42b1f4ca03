"""CPU oracle for the fine-grained FP8 (E4M3) linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
host implementation of what the GPU path computes: the E4M3 codec, the online
max-abs quantizers (1x128 activation tiles, 128x128 weight blocks, 128x1
token-axis tiles, free or power-of-two scales), the block-scaled GEMM in its
dense, grouped and weight-gradient forms, the output acceptance rule, the
accumulation emulators used for the promotion-interval report (written from
the pages' description of limited-width accumulation), and the MoE
glue on either side of the expert GEMMs (FP8 dispatch gather, SwiGLU with
its 1x128 quantization).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library or its
Python binding and imports neither.

Pages cited (they have no titles or section numbers; a citation names the page
address and the paragraph, counted from the top of the page):

* why-be.co.kr wr_id=35533  -- FP8 framework, E4M3 on all tensors
* tmdrlife.com wr_id=13334  -- quantization HBM round trip, fixed-point
  accumulation on Hopper, promotion and scaling, power-of-two scales
* gnrental.net wr_id=40936  -- power-of-two scales, promotion to FP32
* jp-study.kr doc 258368    -- 1x128 / 128x128 online max-abs scaling,
  MoE shapes, FP8 Wgrad, 128-element accumulation interval

Parity status per function is listed in the module docstrings; every function
here is pinned by ``tests/test_oracle_*.py`` except the fixed-point
accumulation emulator beyond its two closed-form special cases, which is
"parity unpinned" (see ``oracle/accum.py``).
"""

from . import e4m3, quantize, gemm, accum, moe  # noqa: F401
