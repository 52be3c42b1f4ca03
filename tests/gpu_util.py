"""Helpers for the GPU parity tests: device transfer of host arrays and a
marker that the native library is loaded (no fallback exists)."""

import sys

import numpy as np
import pytest
import torch

import fine_grained_fp8_fp8q_amd as fp8q


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp8q.load_library()  # raises if libfp8q.so is missing


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(bits):
    """uint16 BF16 patterns (numpy) -> torch.bfloat16 on cuda:0."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host_bf16_bits(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_codes(t):
    """uint8 codes (possibly a padded view) -> dense numpy array."""
    torch.cuda.synchronize()
    return t.contiguous().cpu().numpy()


def assert_codes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first at {tuple(bad[0])}: got {got[tuple(bad[0])]:#04x} want {want[tuple(bad[0])]:#04x}"


def assert_scales_equal(got, want, what):
    g = np.asarray(got, dtype=np.float32).view(np.uint32)
    w = np.asarray(want, dtype=np.float32).view(np.uint32)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    assert bad.size == 0, f"{what}: {len(bad)} scale mismatches, first at {tuple(bad[0])}: got {g[tuple(bad[0])]:#010x} want {w[tuple(bad[0])]:#010x}"
