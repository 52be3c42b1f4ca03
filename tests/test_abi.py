"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status codes before
touching the GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import fine_grained_fp8_fp8q_amd as fp8q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

P16 = ctypes.c_void_p(4096)  # a non-null, 16-byte aligned address (never dereferenced)
P8 = ctypes.c_void_p(4104)   # non-null, not 16-byte aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fp8q.LIB_PATH):
        pytest.skip("libfp8q.so is not built")
    return fp8q.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8q_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_gemm", "fp8q_grouped_gemm", "fp8q_wgrad",
              "fp8q_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(fp8q.SYMBOLS) == _declared()


def test_status_strings(lib):
    for s in range(6):
        assert fp8q.status_string(s)
    assert fp8q.status_string(99) == "unknown status"


def test_quantize_act_validation(lib):
    q = lib.fp8q_quantize_act
    # size 0 -> OK, nothing touched
    assert q(None, 0, 5, 8, 0, 0, None, 16, None, None) == fp8q.OK
    assert q(None, 5, 0, 8, 0, 0, None, 16, None, None) == fp8q.OK
    assert q(None, -1, 5, 8, 0, 0, None, 16, None, None) == fp8q.ERR_INVALID_ARG
    assert q(P16, 4, 8, 8, 2, 0, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG  # bad tile axis
    assert q(P16, 4, 8, 8, 0, 7, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG  # bad scale mode
    assert q(None, 4, 8, 8, 0, 0, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG
    assert q(P16, 4, 16, 8, 0, 0, P16, 16, P16, None) == fp8q.ERR_SHAPE  # ld_x < cols
    assert q(P16, 4, 8, 8, 0, 0, P16, 0, P16, None) == fp8q.ERR_SHAPE  # ld_codes < cols
    assert q(P16, 40, 8, 8, 1, 0, P16, 16, P16, None) == fp8q.ERR_SHAPE  # token_t: ld_codes < rows
    assert q(P8, 4, 8, 8, 0, 0, P16, 16, P16, None) == fp8q.ERR_ALIGN
    assert q(P16, 4, 8, 8, 0, 0, P8, 16, P16, None) == fp8q.ERR_ALIGN
    assert q(P16, 4, 8, 8, 0, 0, P16, 16, P8, None) == fp8q.ERR_ALIGN
    assert q(P16, 1 << 31, 8, 8, 0, 0, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG


def test_quantize_weight_validation(lib):
    q = lib.fp8q_quantize_weight
    assert q(None, 0, 0, 0, 0, None, 0, None, None) == fp8q.OK
    assert q(P16, 4, 8, 8, 3, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG
    assert q(P16, 4, 16, 8, 0, P16, 16, P16, None) == fp8q.ERR_SHAPE
    assert q(P16, 4, 8, 8, 0, P8, 16, P16, None) == fp8q.ERR_ALIGN


def test_gemm_validation(lib):
    # the section 8(b) prototype: (a, sa, w, sw, M, N, K, out_dtype, c, ld_c, stream)
    g = lib.fp8q_gemm
    assert g(None, None, None, None, 0, 4, 128, 0, None, 4, None) == fp8q.OK
    assert g(P16, P16, P16, P16, 4, 4, 100, 0, P16, 4, None) == fp8q.ERR_SHAPE  # K % 128
    assert g(P16, P16, P16, P16, 4, 4, 128, 2, P16, 4, None) == fp8q.ERR_INVALID_ARG
    assert g(None, P16, P16, P16, 4, 4, 128, 0, P16, 4, None) == fp8q.ERR_INVALID_ARG
    assert g(P16, P16, P16, P16, 4, 8, 128, 0, P16, 4, None) == fp8q.ERR_SHAPE  # ld_c < N
    assert g(P16, P16, P16, P16, 4, 4, 128, 1, P8, 4, None) == fp8q.ERR_ALIGN
    assert g(P16, P16, P8, P16, 4, 4, 128, 0, P16, 4, None) == fp8q.ERR_ALIGN
    assert g(P16, P16, P16, P16, 4, 4, -128, 0, P16, 4, None) == fp8q.ERR_INVALID_ARG
    # the _ex form takes acc after out_dtype
    gx = lib.fp8q_gemm_ex
    assert gx(None, None, None, None, 0, 4, 128, 0, 0, None, 4, None) == fp8q.OK
    assert gx(P16, P16, P16, P16, 4, 4, 100, 0, 1, P16, 4, None) == fp8q.ERR_SHAPE
    assert gx(P16, P16, P16, P16, 4, 4, 128, 0, 4, P16, 4, None) == fp8q.ERR_INVALID_ARG  # acc
    assert gx(P16, P16, P16, P16, 4, 4, 128, 0, -1, P16, 4, None) == fp8q.ERR_INVALID_ARG


def test_section_8b_prototypes_in_header():
    """fp8q_gemm, fp8q_grouped_gemm and fp8q_wgrad keep exactly the argument
    lists of the boundary (no accumulation argument); the _ex forms add it."""
    text = " ".join(open(HEADER).read().split())

    def params(name):
        m = re.search(r"fp8q_status " + name + r"\((.*?)\);", text)
        assert m, name
        return [p.strip().split()[-1].lstrip("*") for p in m.group(1).split(",")]

    assert params("fp8q_gemm") == ["a", "a_scales", "w", "w_scales", "M", "N", "K", "out_dtype", "c", "ld_c",
                                   "stream"]
    assert params("fp8q_grouped_gemm") == ["a", "a_scales", "offsets", "G", "rows_cap", "w", "w_scales", "N", "K",
                                           "out_dtype", "c", "ld_c", "stream"]
    assert params("fp8q_wgrad") == ["dy_t", "dy_scales", "x_t", "x_scales", "Nout", "Kin", "T", "dw", "ld_dw",
                                    "stream"]
    assert params("fp8q_gemm_ex") == params("fp8q_gemm")[:8] + ["acc"] + params("fp8q_gemm")[8:]
    assert params("fp8q_grouped_gemm_ex") == (params("fp8q_grouped_gemm")[:10] + ["acc"] +
                                              params("fp8q_grouped_gemm")[10:])
    assert params("fp8q_wgrad_ex") == params("fp8q_wgrad")[:7] + ["acc"] + params("fp8q_wgrad")[7:]


def test_quantize_weight_t_validation(lib):
    q = lib.fp8q_quantize_weight_t
    assert q(None, 0, 8, 8, 0, None, 0, None, None, 0, None, None) == fp8q.OK
    assert q(P16, 4, 8, 8, 0, None, 0, None, None, 16, P16, None) == fp8q.ERR_INVALID_ARG  # codes_t
    assert q(P16, 4, 8, 8, 0, P16, 16, None, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG   # scales
    assert q(P16, 4, 8, 8, 2, None, 0, None, P16, 16, P16, None) == fp8q.ERR_INVALID_ARG   # mode
    assert q(P16, 4, 8, 8, 0, None, 0, None, P16, 3, P16, None) == fp8q.ERR_SHAPE         # ld_codes_t < N
    assert q(P16, 4, 8, 8, 0, P16, 4, P16, P16, 16, P16, None) == fp8q.ERR_SHAPE          # ld_codes < K
    assert q(P16, 4, 8, 8, 0, None, 0, None, P8, 16, P16, None) == fp8q.ERR_ALIGN


def test_grouped_and_wgrad_validation(lib):
    gg = lib.fp8q_grouped_gemm
    assert gg(P16, P16, P16, 0, 10, P16, P16, 4, 128, 0, P16, 4, None) == fp8q.OK  # no groups
    assert gg(P16, P16, P16, -1, 10, P16, P16, 4, 128, 0, P16, 4, None) == fp8q.ERR_INVALID_ARG
    assert gg(P16, P16, None, 2, 10, P16, P16, 4, 128, 0, P16, 4, None) == fp8q.ERR_INVALID_ARG
    assert gg(P16, P16, P16, 2, 10, P16, P16, 4, 64, 0, P16, 4, None) == fp8q.ERR_SHAPE
    assert gg(P16, P16, P8, 2, 10, P16, P16, 4, 128, 0, P16, 4, None) == fp8q.ERR_ALIGN
    ggx = lib.fp8q_grouped_gemm_ex
    assert ggx(P16, P16, P16, 2, 10, P16, P16, 4, 128, 0, 4, P16, 4, None) == fp8q.ERR_INVALID_ARG  # acc
    assert ggx(P16, P16, P16, 2, 10, P16, P16, 4, 64, 0, 1, P16, 4, None) == fp8q.ERR_SHAPE
    wg = lib.fp8q_wgrad
    assert wg(P16, P16, P16, P16, 0, 4, 128, P16, 4, None) == fp8q.OK
    assert wg(P16, P16, P16, P16, 4, 4, 200, P16, 4, None) == fp8q.ERR_SHAPE
    assert wg(P16, P16, P16, P16, 4, 8, 128, P16, 4, None) == fp8q.ERR_SHAPE
    assert wg(P16, None, P16, P16, 4, 4, 128, P16, 4, None) == fp8q.ERR_INVALID_ARG
    wgx = lib.fp8q_wgrad_ex
    assert wgx(P16, P16, P16, P16, 4, 4, 128, 5, P16, 4, None) == fp8q.ERR_INVALID_ARG  # acc
    assert wgx(P16, P16, P16, P16, 4, 4, 200, 2, P16, 4, None) == fp8q.ERR_SHAPE


def test_quantize_linear_validation(lib):
    f = lib.fp8q_quantize_linear
    # (x, M, K, ld_x, amode, a_codes, ld_a, a_scales, w, N, ld_w, wmode, w_codes, ld_wc, w_scales, stream)
    assert f(None, 0, 128, 128, 0, None, 128, None, None, 0, 128, 0, None, 128, None, None) == fp8q.OK
    assert f(P16, 4, 0, 128, 0, P16, 128, P16, P16, 4, 128, 0, P16, 128, P16, None) == fp8q.OK
    assert f(P16, 4, 128, 128, 2, P16, 128, P16, P16, 4, 128, 0, P16, 128, P16, None) == fp8q.ERR_INVALID_ARG
    assert f(P16, 4, 128, 128, 0, P16, 128, P16, P16, 4, 128, 5, P16, 128, P16, None) == fp8q.ERR_INVALID_ARG
    assert f(P16, 4, 128, 128, 0, None, 128, P16, P16, 4, 128, 0, P16, 128, P16, None) == fp8q.ERR_INVALID_ARG
    assert f(P16, 4, 128, 128, 0, P16, 128, P16, P16, 4, 128, 0, P16, 128, None, None) == fp8q.ERR_INVALID_ARG
    assert f(P16, 4, 128, 100, 0, P16, 128, P16, P16, 4, 128, 0, P16, 128, P16, None) == fp8q.ERR_SHAPE
    assert f(P16, 4, 128, 128, 0, P16, 128, P16, P16, 4, 128, 0, P16, 127, P16, None) == fp8q.ERR_SHAPE
    assert f(P8, 4, 128, 128, 0, P16, 128, P16, P16, 4, 128, 0, P16, 128, P16, None) == fp8q.ERR_ALIGN
    assert f(P16, 4, 128, 128, 0, P16, 128, P16, P16, 4, 128, 0, P16, 128, P8, None) == fp8q.ERR_ALIGN
    # one operand may be absent
    assert f(None, 0, 128, 128, 0, None, 128, None, P8, 4, 128, 0, P16, 128, P16, None) == fp8q.ERR_ALIGN


def test_gemm_quantized_validation(lib):
    f = lib.fp8q_gemm_quantized
    # (a, sa, w, sw, M, N, K, acc, scale_mode, codes, ld_c, scales, stream)
    assert f(P16, P16, P16, P16, 0, 4, 128, 0, 0, None, 4, None, None) == fp8q.OK
    assert f(P16, P16, P16, P16, 4, 4, 128, 4, 0, P16, 4, P16, None) == fp8q.ERR_INVALID_ARG  # acc
    assert f(P16, P16, P16, P16, 4, 4, 128, 0, 2, P16, 4, P16, None) == fp8q.ERR_INVALID_ARG  # mode
    assert f(P16, P16, P16, P16, 4, 4, 128, 0, 0, P16, 4, None, None) == fp8q.ERR_INVALID_ARG  # scales
    assert f(P16, P16, P16, P16, 4, 4, 100, 0, 0, P16, 4, P16, None) == fp8q.ERR_SHAPE  # K % 128
    assert f(P16, P16, P16, P16, 4, 8, 128, 0, 0, P16, 4, P16, None) == fp8q.ERR_SHAPE  # ld_c < N
    assert f(P16, P16, P16, P16, 4, 4, 128, 0, 0, P8, 4, P16, None) == fp8q.ERR_ALIGN
    assert f(None, P16, P16, P16, 4, 4, 128, 0, 0, P16, 4, P16, None) == fp8q.ERR_INVALID_ARG


def test_gather_rows_validation(lib):
    g = lib.fp8q_gather_rows
    # (codes, rows, cols, ld_codes, scales, index, n_out, out, ld_out, out_scales, stream)
    assert g(None, 10, 64, 64, None, None, 0, None, 64, None, None) == fp8q.OK  # nothing to write
    assert g(P16, 10, 0, 64, P16, P16, 5, P16, 64, P16, None) == fp8q.OK
    assert g(P16, -1, 64, 64, P16, P16, 5, P16, 64, P16, None) == fp8q.ERR_INVALID_ARG
    assert g(P16, 10, 64, 64, P16, None, 5, P16, 64, P16, None) == fp8q.ERR_INVALID_ARG  # no index
    assert g(None, 10, 64, 64, P16, P16, 5, P16, 64, P16, None) == fp8q.ERR_INVALID_ARG  # no source
    assert g(P16, 10, 64, 32, P16, P16, 5, P16, 64, P16, None) == fp8q.ERR_SHAPE  # ld_codes < cols
    assert g(P16, 10, 64, 64, P16, P16, 5, P16, 63, P16, None) == fp8q.ERR_SHAPE  # ld_out < cols
    assert g(P16, 10, 64, 64, P16, P8, 5, P16, 64, P16, None) == fp8q.ERR_ALIGN
    assert g(P16, 10, 64, 64, P16, P16, 5, P8, 64, P16, None) == fp8q.ERR_ALIGN


def test_swiglu_quantize_validation(lib):
    f = lib.fp8q_swiglu_quantize
    # (x, rows, inter, ld_x, mode, codes, ld_codes, scales, cache_mode, cache_codes, ld_cache, cache_scales, stream)
    assert f(None, 0, 128, 256, 0, None, 128, None, 1, None, 0, None, None) == fp8q.OK
    assert f(P16, 4, 128, 256, 3, P16, 128, P16, 1, None, 0, None, None) == fp8q.ERR_INVALID_ARG  # mode
    assert f(P16, 4, 128, 256, 0, P16, 128, P16, 3, P16, 256, P16, None) == fp8q.ERR_INVALID_ARG  # cache mode
    assert f(P16, 4, 128, 256, 0, None, 128, P16, 1, None, 0, None, None) == fp8q.ERR_INVALID_ARG
    assert f(P16, 4, 128, 256, 0, P16, 128, P16, 1, P16, 256, None, None) == fp8q.ERR_INVALID_ARG  # cache scales
    assert f(P16, 4, 128, 255, 0, P16, 128, P16, 1, None, 0, None, None) == fp8q.ERR_SHAPE  # ld_x < 2*inter
    assert f(P16, 4, 128, 256, 0, P16, 127, P16, 1, None, 0, None, None) == fp8q.ERR_SHAPE
    assert f(P16, 4, 100, 200, 0, P16, 100, P16, 1, P16, 200, P16, None) == fp8q.ERR_SHAPE  # cache: inter % 128
    assert f(P16, 4, 128, 256, 0, P16, 128, P16, 1, P16, 255, P16, None) == fp8q.ERR_SHAPE  # ld_cache
    assert f(P8, 4, 128, 256, 0, P16, 128, P16, 1, None, 0, None, None) == fp8q.ERR_ALIGN
    assert f(P16, 4, 128, 256, 0, P16, 128, P16, 1, P8, 256, P16, None) == fp8q.ERR_ALIGN


def test_valid_calls_reach_the_device_check(lib):
    """Well-formed arguments pass validation; without a gfx950 device the call
    reports FP8Q_ERR_DEVICE and launches nothing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert lib.fp8q_gemm(P16, P16, P16, P16, 4, 4, 128, 0, P16, 4, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_quantize_act(P16, 4, 8, 8, 0, 0, P16, 16, P16, None) == fp8q.ERR_DEVICE
    # leading dimensions need no alignment (unaligned strides take element-wise paths)
    assert lib.fp8q_quantize_act(P16, 4, 7, 7, 0, 0, P16, 7, P16, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_gemm(P16, P16, P16, P16, 4, 5, 128, 1, P16, 5, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_gemm_ex(P16, P16, P16, P16, 4, 5, 128, 1, 1, P16, 5, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_grouped_gemm(P16, P16, P16, 2, 10, P16, P16, 4, 128, 0, P16, 4, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_wgrad(P16, P16, P16, P16, 4, 4, 128, P16, 4, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_wgrad_ex(P16, P16, P16, P16, 4, 4, 128, 2, P16, 4, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_quantize_weight_t(P16, 4, 8, 8, 0, None, 0, None, P16, 16, P16, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_gemm_quantized(P16, P16, P16, P16, 4, 5, 128, 0, 1, P16, 5, P16, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_quantize_linear(P16, 4, 100, 100, 0, P16, 100, P16, P16, 5, 100, 1, P16, 100, P16,
                                    None) == fp8q.ERR_DEVICE
    assert lib.fp8q_quantize_linear(None, 0, 128, 128, 0, None, 128, None, P16, 5, 128, 0, P16, 128, P16,
                                    None) == fp8q.ERR_DEVICE
    assert lib.fp8q_gather_rows(P16, 10, 64, 64, P16, P16, 5, P16, 64, P16, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_gather_rows(None, 0, 64, 64, None, P16, 5, P16, 64, P16, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_swiglu_quantize(P16, 4, 100, 200, 0, P16, 100, P16, 1, None, 0, None, None) == fp8q.ERR_DEVICE
    assert lib.fp8q_swiglu_quantize(P16, 4, 128, 256, 1, P16, 128, P16, 1, P16, 256, P16, None) == fp8q.ERR_DEVICE
