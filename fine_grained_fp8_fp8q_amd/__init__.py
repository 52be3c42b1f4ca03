"""fine_grained_fp8_fp8q_amd -- fine-grained FP8 (E4M3) linear-layer hot path
for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libfp8q.so`` (declared in
``include/fp8q.h``).  Every step of the path runs in the library's HIP
kernels; this module only checks tensor types, allocates outputs with torch
(device memory and the current stream are torch's) and marshals arguments.
There is no fallback: if the library is missing or the device is not gfx950
the calls raise.

Functions (names follow the C ABI without the ``fp8q_`` prefix):

* ``quantize_act(x, tile_axis="row"|"token_t", scale_mode="free"|"pow2")``
  -> (codes uint8, scales float32)
* ``quantize_weight(w, scale_mode="free"|"pow2")`` -> (codes, scales)
* ``quantize_linear(x, w, act_scale_mode=..., weight_scale_mode=...)`` ->
  (a_codes, a_scales, w_codes, w_scales) in one launch
* ``gemm(a, a_scales, w, w_scales, out_dtype=torch.bfloat16|torch.float32)``
* ``grouped_gemm(a, a_scales, offsets, w, w_scales, out_dtype=...)``
* ``wgrad(dy_t, dy_scales, x_t, x_scales)``

  The three GEMMs call ``fp8q_gemm`` / ``fp8q_grouped_gemm`` / ``fp8q_wgrad``
  (partials at float32 grade); ``acc="fp8_mfma"``, ``"fp8_mfma_scaled"`` or
  ``"fp32_pow2"`` calls the ``_ex`` entry point with that accumulation form.
* ``gemm_quantized(a, a_scales, w, w_scales, scale_mode=...)`` -> (codes, scales)
  of C rounded to BF16 and quantized per 1x128 tile along N
* ``gather_rows(codes, scales, index)`` -> (codes, scales) of rows ``index``
* ``swiglu_quantize(x, scale_mode=..., cache=False, cache_scale_mode="pow2")``
  -> (codes, scales[, cache_codes, cache_scales])
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8q.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGN, ERR_LAUNCH, ERR_DEVICE = range(6)
SCALE_FREE, SCALE_POW2 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
ACC_FP32, ACC_FP8_MFMA, ACC_FP8_MFMA_SCALED, ACC_FP32_POW2 = 0, 1, 2, 3
TILE_ROW, TILE_TOKEN_T = 0, 1

SYMBOLS = ("fp8q_quantize_act", "fp8q_quantize_weight", "fp8q_quantize_linear", "fp8q_quantize_weight_t", "fp8q_gemm",
           "fp8q_gemm_ex", "fp8q_gemm_quantized", "fp8q_grouped_gemm", "fp8q_grouped_gemm_ex", "fp8q_wgrad",
           "fp8q_wgrad_ex", "fp8q_gather_rows", "fp8q_swiglu_quantize", "fp8q_set_gemm_small_limit",
           "fp8q_status_string")

_lib = None


class Fp8qError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load_library(path=None):
    """Load libfp8q.so (built in place by ``build.py``) and declare signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m fine_grained_fp8_fp8q_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, i32, ip = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.fp8q_quantize_act.argtypes = [vp, i64, i64, i64, ip, ip, vp, i64, vp, vp]
    lib.fp8q_quantize_weight.argtypes = [vp, i64, i64, i64, ip, vp, i64, vp, vp]
    lib.fp8q_quantize_linear.argtypes = [vp, i64, i64, i64, ip, vp, i64, vp, vp, i64, i64, ip, vp, i64, vp, vp]
    lib.fp8q_quantize_weight_t.argtypes = [vp, i64, i64, i64, ip, vp, i64, vp, vp, i64, vp, vp]
    lib.fp8q_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, ip, vp, i64, vp]
    lib.fp8q_gemm_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, ip, ip, vp, i64, vp]
    lib.fp8q_gemm_quantized.argtypes = [vp, vp, vp, vp, i64, i64, i64, ip, ip, vp, i64, vp, vp]
    lib.fp8q_grouped_gemm.argtypes = [vp, vp, vp, i32, i64, vp, vp, i64, i64, ip, vp, i64, vp]
    lib.fp8q_grouped_gemm_ex.argtypes = [vp, vp, vp, i32, i64, vp, vp, i64, i64, ip, ip, vp, i64, vp]
    lib.fp8q_wgrad.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.fp8q_wgrad_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, ip, vp, i64, vp]
    lib.fp8q_gather_rows.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, i64, vp, vp]
    lib.fp8q_swiglu_quantize.argtypes = [vp, i64, i64, i64, ip, vp, i64, vp, ip, vp, i64, vp, vp]
    lib.fp8q_set_gemm_small_limit.argtypes = [i64]
    lib.fp8q_set_gemm_small_limit.restype = i64
    for name in SYMBOLS[:-2]:
        getattr(lib, name).restype = ctypes.c_int
    lib.fp8q_status_string.argtypes = [ctypes.c_int]
    lib.fp8q_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status):
    return load_library().fp8q_status_string(int(status)).decode()


def _check(status, where):
    if status != OK:
        raise Fp8qError(status, where)


# ------------------------------------------------------- torch plumbing ----

def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _row_major(t, name):
    """Row stride of a 2-D tensor with contiguous rows (any stride is fine for
    an empty one: nothing is read through it)."""
    if t.dim() != 2 or (t.numel() and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    return t.stride(0) if t.numel() else max(t.shape[1], 1)


def _pad16(n):
    return (n + 15) // 16 * 16


def _scale_mode(mode):
    return {"free": SCALE_FREE, "pow2": SCALE_POW2}[mode]


def _alloc_codes(rows, cols, device):
    """uint8 [rows, cols] view of a buffer whose row stride is a multiple of 16."""
    torch = _torch()
    buf = torch.empty((rows, _pad16(max(cols, 1))), dtype=torch.uint8, device=device)
    return buf[:, :cols]


# ------------------------------------------------------------ the calls ----

def quantize_act(x, tile_axis="row", scale_mode="free"):
    """BF16 [rows, cols] -> (codes, scales).

    tile_axis="row": 1x128 tiles along cols; codes [rows, cols],
    scales [rows, ceil(cols/128)].  tile_axis="token_t": 128x1 tiles along
    rows; codes [cols, rows] (transposed), scales [cols, ceil(rows/128)].
    """
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    ldx = _row_major(x, "x")
    rows, cols = x.shape
    axis = {"row": TILE_ROW, "token_t": TILE_TOKEN_T}[tile_axis]
    if axis == TILE_ROW:
        codes = _alloc_codes(rows, cols, x.device)
        scales = torch.empty((rows, (cols + 127) // 128), dtype=torch.float32, device=x.device)
    else:
        codes = _alloc_codes(cols, rows, x.device)
        scales = torch.empty((cols, (rows + 127) // 128), dtype=torch.float32, device=x.device)
    st = load_library().fp8q_quantize_act(_ptr(x), rows, cols, ldx, axis, _scale_mode(scale_mode),
                                          _ptr(codes), codes.stride(0) if codes.numel() else 16,
                                          _ptr(scales), _stream(x))
    _check(st, "fp8q_quantize_act")
    return codes, scales


def quantize_weight(w, scale_mode="free"):
    """BF16 [N, K] -> (codes [N, K], scales [ceil(N/128), ceil(K/128)])."""
    torch = _torch()
    _need(w, torch.bfloat16, "w")
    ldw = _row_major(w, "w")
    n, k = w.shape
    codes = _alloc_codes(n, k, w.device)
    scales = torch.empty(((n + 127) // 128, (k + 127) // 128), dtype=torch.float32, device=w.device)
    st = load_library().fp8q_quantize_weight(_ptr(w), n, k, ldw, _scale_mode(scale_mode), _ptr(codes),
                                             codes.stride(0) if codes.numel() else 16, _ptr(scales),
                                             _stream(w))
    _check(st, "fp8q_quantize_weight")
    return codes, scales


def quantize_linear(x, w, act_scale_mode="free", weight_scale_mode="free"):
    """Both operands of a linear layer in one launch: the activation x
    [M, K] per 1x128 tile and the weight w [N, K] per 128x128 block, bit for
    bit ``quantize_act(x)`` and ``quantize_weight(w)``."""
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    _need(w, torch.bfloat16, "w")
    ldx = _row_major(x, "x")
    ldw = _row_major(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("x and w must have the same K")
    nb = (k + 127) // 128
    ac = _alloc_codes(m, k, x.device)
    as_ = torch.empty((m, nb), dtype=torch.float32, device=x.device)
    wc = _alloc_codes(n, k, x.device)
    ws = torch.empty(((n + 127) // 128, nb), dtype=torch.float32, device=x.device)
    st = load_library().fp8q_quantize_linear(
        _ptr(x), m, k, ldx if x.numel() else k, _scale_mode(act_scale_mode), _ptr(ac),
        ac.stride(0) if ac.numel() else _pad16(max(k, 1)), _ptr(as_), _ptr(w), n, ldw if w.numel() else k,
        _scale_mode(weight_scale_mode), _ptr(wc), wc.stride(0) if wc.numel() else _pad16(max(k, 1)), _ptr(ws),
        _stream(x))
    _check(st, "fp8q_quantize_linear")
    return ac, as_, wc, ws


def quantize_weight_t(w, scale_mode="free", both=True):
    """BF16 [N, K] -> (codes, scales, codes_t, scales_t): the 128x128 block
    quantization of w and its transpose (codes_t [K, N], scales_t
    [ceil(K/128), ceil(N/128)]) from one pass; with both=False only the
    transposed pair is written and codes, scales are None.  The transposed
    pair is the W operand of the activation-gradient GEMM (see dgrad)."""
    torch = _torch()
    _need(w, torch.bfloat16, "w")
    ldw = _row_major(w, "w")
    n, k = w.shape
    codes = _alloc_codes(n, k, w.device) if both else None
    scales = torch.empty(((n + 127) // 128, (k + 127) // 128), dtype=torch.float32, device=w.device) \
        if both else None
    codes_t = _alloc_codes(k, n, w.device)
    scales_t = torch.empty(((k + 127) // 128, (n + 127) // 128), dtype=torch.float32, device=w.device)
    st = load_library().fp8q_quantize_weight_t(
        _ptr(w), n, k, ldw, _scale_mode(scale_mode),
        _ptr(codes) if both else None, (codes.stride(0) if codes.numel() else 16) if both else 16,
        _ptr(scales) if both else None,
        _ptr(codes_t), codes_t.stride(0) if codes_t.numel() else 16, _ptr(scales_t), _stream(w))
    _check(st, "fp8q_quantize_weight_t")
    return codes, scales, codes_t, scales_t


def _out_code(dtype):
    torch = _torch()
    if dtype == torch.bfloat16:
        return OUT_BF16
    if dtype == torch.float32:
        return OUT_F32
    raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")


def _acc_code(acc):
    """"fp32" (default; partials at float32 grade), "fp8_mfma" (partials
    formed inside the FP8 matrix core, ~14-bit alignment in groups of 8),
    "fp8_mfma_scaled" (power-of-two scales applied by the matrix core, all K
    blocks accumulated there: no promotion) or "fp32_pow2" (power-of-two
    scales applied exactly while widening to BF16, float32 grade, all K
    blocks accumulated in the BF16 matrix core: no fold)."""
    try:
        return {"fp32": ACC_FP32, "fp8_mfma": ACC_FP8_MFMA, "fp8_mfma_scaled": ACC_FP8_MFMA_SCALED,
                "fp32_pow2": ACC_FP32_POW2}[acc]
    except KeyError:
        raise ValueError('acc must be "fp32", "fp8_mfma", "fp8_mfma_scaled" or "fp32_pow2"') from None


def _contig_codes(t, name):
    torch = _torch()
    _need(t, torch.uint8, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (K-contiguous rows, no padding)")


def _contig_f32(t, name):
    torch = _torch()
    _need(t, torch.float32, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gemm(a, a_scales, w, w_scales, out_dtype=None, out=None, acc="fp32"):
    """C[M, N] = block-scaled A . W^T from E4M3 codes and float32 scales."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    for t, n in ((a, "a"), (w, "w")):
        _contig_codes(t, n)
    for t, n in ((a_scales, "a_scales"), (w_scales, "w_scales")):
        _contig_f32(t, n)
    m, k = a.shape
    n = w.shape[0]
    if w.shape[1] != k or a_scales.shape != (m, k // 128) or w_scales.shape != ((n + 127) // 128, k // 128):
        raise ValueError("operand shapes do not match")
    c = out if out is not None else torch.empty((m, n), dtype=out_dtype, device=a.device)
    lib, code = load_library(), _acc_code(acc)
    if code == ACC_FP32:
        st = lib.fp8q_gemm(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales), m, n, k, _out_code(c.dtype), _ptr(c),
                           c.stride(0), _stream(a))
    else:
        st = lib.fp8q_gemm_ex(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales), m, n, k, _out_code(c.dtype), code,
                              _ptr(c), c.stride(0), _stream(a))
    _check(st, "fp8q_gemm")
    return c


def set_gemm_small_limit(max_outputs):
    """Outputs (M * N) up to which the float32-grade dense GEMM uses 32 x 32
    split-K tiles; a negative value restores the default.  Returns the
    previous setting (-1 for the default)."""
    return int(load_library().fp8q_set_gemm_small_limit(int(max_outputs)))


def gemm_quantized(a, a_scales, w, w_scales, scale_mode="free", acc="fp32"):
    """C = A . W^T (as ``gemm``) rounded to BF16 and quantized per 1x128
    tile along N in the epilogue: (codes uint8 [M, N], scales float32
    [M, ceil(N/128)]), bit for bit ``quantize_act(gemm(..., bfloat16))``."""
    torch = _torch()
    _contig_codes(a, "a")
    _contig_codes(w, "w")
    _contig_f32(a_scales, "a_scales")
    _contig_f32(w_scales, "w_scales")
    m, k = a.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("a and w must have the same K")
    codes = _alloc_codes(m, n, a.device)
    scales = torch.empty((m, (n + 127) // 128), dtype=torch.float32, device=a.device)
    st = load_library().fp8q_gemm_quantized(_ptr(a), _ptr(a_scales), _ptr(w), _ptr(w_scales), m, n, k,
                                            _acc_code(acc), _scale_mode(scale_mode), _ptr(codes),
                                            codes.stride(0) if codes.numel() else _pad16(max(n, 1)),
                                            _ptr(scales), _stream(a))
    _check(st, "fp8q_gemm_quantized")
    return codes, scales


def dgrad(dy, dy_scales, w_t, w_t_scales, out_dtype=None, out=None, acc="fp32"):
    """dX[M, K] = dY[M, N] . W[N, K] from dY quantized in 1x128 tiles along N
    and the transposed weight pair of quantize_weight_t: the block-scaled
    GEMM with reduction axis N (fp8q_gemm on those operands)."""
    return gemm(dy, dy_scales, w_t, w_t_scales, out_dtype=out_dtype, out=out, acc=acc)


def grouped_gemm(a, a_scales, offsets, w, w_scales, out_dtype=None, out=None, acc="fp32"):
    """Per-expert block-scaled GEMM; rows [offsets[g], offsets[g+1]) use w[g].

    offsets: int32 device tensor [G+1].  Rows of the output not covered by any
    group are left as allocated (uninitialised unless ``out`` is given).
    """
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _contig_codes(a, "a")
    _contig_codes(w, "w")
    _contig_f32(a_scales, "a_scales")
    _contig_f32(w_scales, "w_scales")
    _need(offsets, torch.int32, "offsets")
    rows_cap, k = a.shape
    g, n, kw = w.shape
    if kw != k or offsets.numel() != g + 1:
        raise ValueError("operand shapes do not match")
    c = out if out is not None else torch.empty((rows_cap, n), dtype=out_dtype, device=a.device)
    lib, code = load_library(), _acc_code(acc)
    if code == ACC_FP32:
        st = lib.fp8q_grouped_gemm(_ptr(a), _ptr(a_scales), _ptr(offsets), g, rows_cap, _ptr(w), _ptr(w_scales), n,
                                   k, _out_code(c.dtype), _ptr(c), c.stride(0), _stream(a))
    else:
        st = lib.fp8q_grouped_gemm_ex(_ptr(a), _ptr(a_scales), _ptr(offsets), g, rows_cap, _ptr(w),
                                      _ptr(w_scales), n, k, _out_code(c.dtype), code, _ptr(c), c.stride(0),
                                      _stream(a))
    _check(st, "fp8q_grouped_gemm")
    return c


def wgrad(dy_t, dy_scales, x_t, x_scales, out=None, acc="fp32"):
    """dW[Nout, Kin] = dY^T X (float32) from token-axis-quantized operands."""
    torch = _torch()
    _contig_codes(dy_t, "dy_t")
    _contig_codes(x_t, "x_t")
    _contig_f32(dy_scales, "dy_scales")
    _contig_f32(x_scales, "x_scales")
    nout, t = dy_t.shape
    kin = x_t.shape[0]
    if x_t.shape[1] != t:
        raise ValueError("operand shapes do not match")
    dw = out if out is not None else torch.empty((nout, kin), dtype=torch.float32, device=dy_t.device)
    lib, code = load_library(), _acc_code(acc)
    if code == ACC_FP32:
        st = lib.fp8q_wgrad(_ptr(dy_t), _ptr(dy_scales), _ptr(x_t), _ptr(x_scales), nout, kin, t, _ptr(dw),
                            dw.stride(0), _stream(dy_t))
    else:
        st = lib.fp8q_wgrad_ex(_ptr(dy_t), _ptr(dy_scales), _ptr(x_t), _ptr(x_scales), nout, kin, t, code,
                               _ptr(dw), dw.stride(0), _stream(dy_t))
    _check(st, "fp8q_wgrad")
    return dw


def gather_rows(codes, scales, index):
    """FP8 dispatch gather: (codes[index], scales[index]) as new tensors.

    codes uint8 [rows, cols] with contiguous rows (e.g. ``quantize_act``
    output), scales float32 [rows, ceil(cols/128)] contiguous, index int32
    [n] on the GPU.  An index outside [0, rows) yields a zero row and a zero
    scale (the library does not check indices on the host).
    """
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    ldc = _row_major(codes, "codes")
    _contig_f32(scales, "scales")
    _need(index, torch.int32, "index")
    if index.dim() != 1 or not index.is_contiguous():
        raise ValueError("index must be a contiguous 1-D int32 tensor")
    rows, cols = codes.shape
    nb = (cols + 127) // 128
    if tuple(scales.shape) != (rows, nb):
        raise ValueError(f"scales must be [{rows}, {nb}], got {tuple(scales.shape)}")
    n = index.numel()
    out = _alloc_codes(n, cols, codes.device)
    out_s = torch.empty((n, nb), dtype=torch.float32, device=codes.device)
    st = load_library().fp8q_gather_rows(_ptr(codes), rows, cols, ldc if codes.numel() else cols,
                                         _ptr(scales), _ptr(index), n, _ptr(out),
                                         out.stride(0) if out.numel() else _pad16(max(cols, 1)),
                                         _ptr(out_s), _stream(codes))
    _check(st, "fp8q_gather_rows")
    return out, out_s


def swiglu_quantize(x, scale_mode="free", cache=False, cache_scale_mode="pow2"):
    """SwiGLU of x = [gate | up] (BF16 [rows, 2*inter]), quantized 1x128.

    Returns (codes [rows, inter], scales [rows, ceil(inter/128)]); with
    cache=True also the 1x128 quantization of x itself (cache_scale_mode,
    inter a multiple of 128): (codes, scales, cache_codes [rows, 2*inter],
    cache_scales [rows, 2*inter/128]).
    """
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    ldx = _row_major(x, "x")
    rows, two_inter = x.shape
    if two_inter % 2:
        raise ValueError("x must have an even number of columns (gate | up)")
    inter = two_inter // 2
    codes = _alloc_codes(rows, inter, x.device)
    scales = torch.empty((rows, (inter + 127) // 128), dtype=torch.float32, device=x.device)
    cc = cs = None
    if cache:
        cc = _alloc_codes(rows, two_inter, x.device)
        cs = torch.empty((rows, (two_inter + 127) // 128), dtype=torch.float32, device=x.device)
    st = load_library().fp8q_swiglu_quantize(
        _ptr(x), rows, inter, ldx if x.numel() else two_inter, _scale_mode(scale_mode), _ptr(codes),
        codes.stride(0) if codes.numel() else _pad16(max(inter, 1)), _ptr(scales),
        _scale_mode(cache_scale_mode), _ptr(cc) if cache else ctypes.c_void_p(0),
        cc.stride(0) if cache and cc.numel() else _pad16(max(two_inter, 1)),
        _ptr(cs) if cache else ctypes.c_void_p(0), _stream(x))
    _check(st, "fp8q_swiglu_quantize")
    return (codes, scales, cc, cs) if cache else (codes, scales)
