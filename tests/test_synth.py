"""The seeded input generators: shapes, determinism, BF16 rounding."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * np.exp2(rng.uniform(-60, 60, 50000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_rne(x), ref)


def test_tiny_linear_recipe():
    d1, d2 = synth.tiny_linear(), synth.tiny_linear()
    assert d1["a"].shape == (128, 512) and d1["w"].shape == (256, 512)
    assert np.array_equal(d1["a"], d2["a"]) and np.array_equal(d1["w"], d2["w"])
    a = (d1["a"].astype(np.uint32) << 16).view(np.float32)
    assert 280 <= (np.abs(a) > 5).sum() <= 328  # the 328 outliers x50 make the tail
    w = (d1["w"].astype(np.uint32) << 16).view(np.float32)
    assert 0.018 < w.std() < 0.022


def test_moe_routing_has_an_empty_group_and_is_seeded():
    l1, c1 = synth.moe_routing()
    l2, c2 = synth.moe_routing()
    assert np.array_equal(c1, c2) and (c1 == 0).sum() >= 1
    assert all(np.all(np.diff(v) > 0) for v in l1)
    assert c1.max() <= 8192


def test_random_codes_and_scales():
    rng = np.random.default_rng(3)
    c = synth.e4m3_codes(rng, (512, 1024))
    counts = np.bincount(c.ravel(), minlength=256)
    assert c.dtype == np.uint8 and c.shape == (512, 1024)
    assert counts[0x7F] == 0 and counts[0xFF] == 0       # no NaN pattern
    assert (counts[[b for b in range(256) if b & 0x7F != 0x7F]] > 0).all()  # every finite code drawn
    assert np.array_equal(c, synth.e4m3_codes(np.random.default_rng(3), (512, 1024)))
    s = synth.tile_scales(rng, (1000, 56))
    assert s.dtype == np.float32 and (s >= 2.0 ** -8).all() and (s < 2.0 ** 8).all()
    assert np.unique(s).size > 50000                      # free mantissas, not powers of two
