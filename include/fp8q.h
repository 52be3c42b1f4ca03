/*
 * fp8q -- fine-grained FP8 (E4M3) quantization and block-scaled GEMM for
 * AMD Instinct MI355X (gfx950).  C ABI of libfp8q.so.
 *
 * What the library computes (pages cited by address and paragraph; they carry
 * no titles or section numbers):
 *
 *  - why-be.co.kr wr_id=35533 ¶2: every GEMM operand is E4M3 (4-bit exponent,
 *    3-bit mantissa).  The OCP variant is used: bias 7, largest finite 448,
 *    NaN at S.1111.111, no infinities.
 *  - jp-study.kr doc 258368 ¶1: scaling is online max-abs, per 1x128
 *    activation tile and per 128x128 weight block.  A tile's scale is
 *    s = RN32(amax / 448) and an element's code is E4M3_RNE(RN32(x / s))
 *    (IEEE float32 division, then round-to-nearest-even to E4M3, saturating
 *    at +-448, sign of zero kept).  An all-zero tile gets s = 0 and signed
 *    zero codes.
 *  - tmdrlife.com wr_id=13334 ¶4, gnrental.net wr_id=40936 ¶3: some
 *    activations use power-of-two scales: s = the smallest 2^e with
 *    amax / s <= 448, so x / s is exact.
 *  - tmdrlife.com wr_id=13334 ¶3, gnrental.net wr_id=40936 ¶4, jp-study.kr
 *    doc 258368 ¶3: the GEMM forms FP8 partial products over 128 elements of
 *    K, then multiplies each partial by its activation and weight scales and
 *    adds it into FP32 accumulators:
 *        C[m,n] = sum_b a_scales[m,b] * w_scales[n/128,b] * sum_{k in b} A[m,k] W[n,k]
 *  - jp-study.kr doc 258368 ¶3: the weight gradient (Wgrad) runs in FP8 too;
 *    its reduction axis is the token axis, so both operands are quantized in
 *    128-token x 1-feature tiles.
 *
 * Conventions for every call:
 *  - Memory: all pointers are DEVICE pointers owned by the caller.  The
 *    library allocates nothing, frees nothing and keeps no pointer after
 *    the call returns.
 *  - Execution: work is enqueued on `stream` (0 = the null stream) and the
 *    call returns without synchronizing.  There is no global mutable state
 *    beyond a per-device architecture check cached on first use, so calls
 *    are re-entrant and thread-safe.
 *  - Errors: argument errors are detected before anything is launched; the
 *    outputs are then untouched.  A failed launch returns FP8Q_ERR_LAUNCH.
 *    Faults inside kernels surface at the caller's next synchronization.
 *    A current device that is not gfx950 gives FP8Q_ERR_DEVICE.
 *  - Sizes: int64 values, each below 2^31.  Zero-sized outputs return
 *    FP8Q_OK without launching.  Inputs must be finite.
 *  - Alignment: every base pointer must be 16-byte aligned (FP8Q_ERR_ALIGN
 *    otherwise).  Leading dimensions (in elements) only need to be at least
 *    the row length; strides that break 16-byte row alignment are accepted
 *    and take slower element-wise load/store paths.
 *  - Aliasing between inputs and outputs is not allowed.
 *  - BF16 data is passed as raw 16-bit patterns; codes are uint8 E4M3
 *    patterns; scales are float32, always densely packed (no leading dim).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

typedef enum fp8q_status {
  FP8Q_OK = 0,
  FP8Q_ERR_INVALID_ARG = 1, /* null pointer, negative size, unknown enum value */
  FP8Q_ERR_SHAPE = 2,       /* leading dim below the row length, K not a multiple of 128, size >= 2^31 */
  FP8Q_ERR_ALIGN = 3,       /* a base pointer is not 16-byte aligned */
  FP8Q_ERR_LAUNCH = 4,      /* the HIP runtime rejected a kernel launch */
  FP8Q_ERR_DEVICE = 5       /* no current device, or it is not gfx950 */
} fp8q_status;

enum { FP8Q_SCALE_FREE = 0, FP8Q_SCALE_POW2 = 1 };
enum { FP8Q_OUT_F32 = 0, FP8Q_OUT_BF16 = 1 };
/* How each 128-element partial sum of E4M3 products is formed before it is
 * scaled and added into the FP32 accumulators (tmdrlife.com wr_id=13334 ¶2-¶3,
 * why-be.co.kr wr_id=35533 ¶4: the FP8 matrix unit keeps its running sum in a
 * limited width; promotion every 128 elements bounds the damage).
 *  FP8Q_ACC_FP32: the partial is formed at float32 grade (operands widened
 *    exactly to BF16, BF16 matrix-core products and float32 sums).  Results
 *    satisfy |C - exact| <= 1e-5 * sum|a*b| + 1e-6.
 *  FP8Q_ACC_FP8_MFMA: the partial is formed by the FP8 matrix core itself
 *    (v_mfma_f32_16x16x128_f8f6f4), twice the FP32 form's throughput.  Measured
 *    on MI355X: within each aligned group of 8 consecutive products, every
 *    product is truncated toward zero to a multiple of 2^(E-13), E being the
 *    exponent of the group's largest product; group sums are then added at
 *    about float32 grade.  The error of a partial is therefore below
 *    sum over its 16 groups of 8 * 2^(E_g - 13) plus float32 rounding, and
 *    can exceed the FP32 form's bound when one product dominates its group.
 *  FP8Q_ACC_FP8_MFMA_SCALED: for power-of-two scales only (FP8Q_SCALE_POW2
 *    on both operands, every scale in [2^-127, 2^127] or zero): the scales'
 *    exponents are handed to v_mfma_scale_f32_16x16x128_f8f6f4 as E8M0 block
 *    scales, so the matrix core applies them itself (tmdrlife.com
 *    wr_id=13334 ¶3: MMA with group scaling) and every K block accumulates
 *    in the matrix core's accumulator: no VALU fold and no promotion; the
 *    in-group alignment of FP8Q_ACC_FP8_MFMA applies, and the running sum
 *    is added to at about float32 grade once per group of 8 products.
 *    A scale that is not a power of two is used as the power of two of its
 *    exponent (results are then wrong).
 *  FP8Q_ACC_FP32_POW2: for power-of-two scales only (FP8Q_SCALE_POW2 on both
 *    operands), float32 grade like FP8Q_ACC_FP32: each operand is widened to
 *    BF16 with its scale applied by the convert (an E4M3 value times 2^e is
 *    again a BF16 value), so every BF16 matrix-core product is
 *    sa * sw * a * w exactly and all K blocks accumulate in the matrix
 *    core's float32 accumulator (tmdrlife.com wr_id=13334 ¶3-¶4: MMA with
 *    group scaling, integral power-of-two scales): no VALU fold.  Results
 *    satisfy the FP8Q_ACC_FP32 bound while every scaled operand stays in
 *    BF16's normal range (scales in [2^-100, 2^100] or zero, which power-of-
 *    two quantization of BF16 values with max-abs >= 2^-92 gives); scales
 *    that are not powers of two give wrong results. */
enum { FP8Q_ACC_FP32 = 0, FP8Q_ACC_FP8_MFMA = 1, FP8Q_ACC_FP8_MFMA_SCALED = 2, FP8Q_ACC_FP32_POW2 = 3 };
enum {
  FP8Q_TILE_ROW = 0,    /* 1x128 tiles along cols: codes [rows, ld_codes], scales [rows, ceil(cols/128)] */
  FP8Q_TILE_TOKEN_T = 1 /* 128x1 tiles along rows (the token axis), codes written transposed:
                           codes [cols, ld_codes] with ld_codes >= rows, scales [cols, ceil(rows/128)] */
};

/* Quantize a BF16 activation x[rows, cols] (row stride ld_x elements) into
 * E4M3 codes and float32 scales with online max-abs scaling per tile
 * (jp-study.kr doc 258368 ¶1; power-of-two mode: tmdrlife.com wr_id=13334 ¶4).
 * tile_axis: FP8Q_TILE_ROW (1x128 along the GEMM reduction axis, the last
 * tile of a row may be ragged) or FP8Q_TILE_TOKEN_T (128x1 along rows; the
 * output is feature-major so a token-axis GEMM reads it K-contiguous).
 * scale_mode: FP8Q_SCALE_FREE or FP8Q_SCALE_POW2.  Codes outside the valid
 * region of each output row are not written.  Token tiles: fewer than 2^24
 * workgroups of 128 tokens x 64 features, else FP8Q_ERR_SHAPE (no input
 * that fits in device memory reaches it). */
fp8q_status fp8q_quantize_act(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int tile_axis, int scale_mode,
                              uint8_t* codes, int64_t ld_codes, float* scales,
                              hipStream_t stream);

/* Quantize a BF16 weight w[N, K] (row stride ld_w elements) per 128x128
 * block (jp-study.kr doc 258368 ¶1).  codes [N, ld_codes];
 * scales [ceil(N/128), ceil(K/128)] row-major.  Edge blocks may be ragged in
 * both directions.  Fewer than 2^23 blocks (one workgroup each), else
 * FP8Q_ERR_SHAPE; the same bound holds for fp8q_quantize_linear and
 * fp8q_quantize_weight_t. */
fp8q_status fp8q_quantize_weight(const void* w_bf16, int64_t N, int64_t K, int64_t ld_w,
                                 int scale_mode,
                                 uint8_t* codes, int64_t ld_codes, float* scales,
                                 hipStream_t stream);

/* Both operands of a linear layer in one launch: the activation x [M, K]
 * exactly as fp8q_quantize_act(FP8Q_TILE_ROW, act_scale_mode) quantizes it
 * (a_codes [M, ld_a >= K], a_scales [M, ceil(K/128)]) and the weight w [N, K]
 * exactly as fp8q_quantize_weight(weight_scale_mode) quantizes it (w_codes
 * [N, ld_wc >= K], w_scales [ceil(N/128), ceil(K/128)]) -- the online
 * scaling of jp-study.kr doc 258368 ¶1 for the two inputs of one FP8 GEMM,
 * with one grid ramp and drain instead of two.  M or N may be 0 (that
 * operand is skipped; its pointers may then be NULL). */
fp8q_status fp8q_quantize_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ld_x, int act_scale_mode,
                                 uint8_t* a_codes, int64_t ld_a, float* a_scales,
                                 const void* w_bf16, int64_t N, int64_t ld_w, int weight_scale_mode,
                                 uint8_t* w_codes, int64_t ld_wc, float* w_scales, hipStream_t stream);

/* The quantization of fp8q_quantize_weight, written for the activation
 * gradient too (jp-study.kr doc 258368 ¶3: Fprop, Dgrad and Wgrad all take
 * FP8 inputs).  dX[M,K] = dY[M,N] . W[N,K] reduces over N, so it needs W^T
 * with N contiguous; a 128x128 block's max-abs does not depend on
 * orientation, so W^T quantized per block is exactly the transpose of W
 * quantized, and dX = fp8q_gemm(dY codes, dY scales, codes_t, scales_t) with
 * dY quantized in 1x128 tiles along N.
 * codes_t [K, ld_codes_t >= N]; scales_t [ceil(K/128), ceil(N/128)] with
 * scales_t[j][i] = the scale of block (i, j).  codes/scales (as for
 * fp8q_quantize_weight) may both be NULL, then only the transposed copy is
 * written; otherwise both copies come from one read of w. */
fp8q_status fp8q_quantize_weight_t(const void* w_bf16, int64_t N, int64_t K, int64_t ld_w,
                                   int scale_mode,
                                   uint8_t* codes, int64_t ld_codes, float* scales,
                                   uint8_t* codes_t, int64_t ld_codes_t, float* scales_t,
                                   hipStream_t stream);

/* Block-scaled GEMM C[M,N] = A . W^T (tmdrlife.com wr_id=13334 ¶3;
 * jp-study.kr doc 258368 ¶3):
 *   C[m,n] = sum_b a_scales[m,b] * w_scales[n/128,b] * sum_{k in block b} A[m,k] * W[n,k]
 * a: codes [M, K] contiguous; a_scales [M, K/128]; w: codes [N, K]
 * contiguous; w_scales [ceil(N/128), K/128].  K must be a multiple of 128
 * (K = 0 writes zeros).  out_dtype FP8Q_OUT_F32 (c is float*) or
 * FP8Q_OUT_BF16 (c holds BF16 patterns, rounded to nearest even); row
 * stride ld_c elements.  C is overwritten.  Partials are formed at float32
 * grade (FP8Q_ACC_FP32): |C - exact| <= 1e-5 * sum|a*b| + 1e-6.
 * Each code operand is below 2 GiB, and fewer than 2^23 output tiles of
 * 256 x 224 (one workgroup each: tiles are 256 or 224 columns wide,
 * whichever fills the compute units in fewer column-widths; for the grouped
 * form the tile count it launches), else FP8Q_ERR_SHAPE. */
fp8q_status fp8q_gemm(const uint8_t* a, const float* a_scales,
                      const uint8_t* w, const float* w_scales,
                      int64_t M, int64_t N, int64_t K, int out_dtype,
                      void* c, int64_t ld_c, hipStream_t stream);

/* Tiling of the dense float32-grade GEMM (fp8q_gemm, and fp8q_gemm_ex with
 * FP8Q_ACC_FP32), for outputs too small to fill the compute units with
 * 256-wide tiles (a linear layer over a few hundred tokens): an output of at
 * most max_outputs elements (M * N) runs on 32 x 32 tiles whose K blocks are
 * split over the four waves of a workgroup and added in a fixed order;
 * larger outputs run on 256 x 256 (or 256 x 224) tiles, each over the whole
 * of K.  Both satisfy the bound stated for fp8q_gemm; they may differ from
 * each other by the float32 rounding of the summation order.  The other
 * accumulation forms always take the large tiles.  Default, and after any
 * negative value: 8192 outputs per compute unit of the device a launch runs
 * on (as many outputs as an eighth of the compute units hold in 256 x 256
 * tiles).  Process-wide and atomic; launches issued after the call see the
 * new value.  Returns the previous setting (-1 for the default). */
int64_t fp8q_set_gemm_small_limit(int64_t max_outputs);

/* fp8q_gemm with the accumulation form chosen by the caller: acc is one of
 * the FP8Q_ACC_* values above (fp8q_gemm is fp8q_gemm_ex with
 * FP8Q_ACC_FP32).  Same arguments, layouts and errors otherwise; an unknown
 * acc gives FP8Q_ERR_INVALID_ARG. */
fp8q_status fp8q_gemm_ex(const uint8_t* a, const float* a_scales,
                         const uint8_t* w, const float* w_scales,
                         int64_t M, int64_t N, int64_t K, int out_dtype, int acc,
                         void* c, int64_t ld_c, hipStream_t stream);

/* fp8q_gemm with its output quantized in the epilogue, for a consumer that
 * takes FP8 input (tmdrlife.com wr_id=13334 ¶1: the BF16 output of one
 * computation is read back from HBM only to be quantized, written as FP8 and
 * read again for the next MMA; here the producer writes the FP8 form
 * directly).  C is formed exactly as fp8q_gemm forms it on 256-wide tiles
 * (acc as there), rounded to BF16 (nearest even) as with FP8Q_OUT_BF16, and
 * that BF16 tensor is quantized per 1x128 tile along N exactly as
 * fp8q_quantize_act (FP8Q_TILE_ROW, scale_mode) quantizes it: the result is
 * bit for bit the unfused fp8q_gemm(FP8Q_OUT_BF16) -- on 256-wide tiles,
 * which it takes for every output larger than the limit of
 * fp8q_set_gemm_small_limit -- followed by fp8q_quantize_act, without the
 * BF16 round trip through HBM.
 * a, a_scales, w, w_scales, M, N, K as for fp8q_gemm, acc as for fp8q_gemm_ex; c_codes
 * [M, ld_c >= N] E4M3; c_scales [M, ceil(N/128)] float32. */
fp8q_status fp8q_gemm_quantized(const uint8_t* a, const float* a_scales,
                                const uint8_t* w, const float* w_scales,
                                int64_t M, int64_t N, int64_t K, int acc, int scale_mode,
                                uint8_t* c_codes, int64_t ld_c, float* c_scales, hipStream_t stream);

/* Grouped block-scaled GEMM for the MoE experts one device hosts
 * (jp-study.kr doc 258368 ¶1-¶2: activations quantized before the expert
 * dispatch; each device hosts several experts).  Rows
 * [offsets[g], offsets[g+1]) of a use expert g's weights w[g]:
 *   C[r,n] = sum_b a_scales[r,b] * w_scales[g, n/128, b] * sum_k A[r,k] * W[g,n,k]
 * a: codes [rows_cap, K]; a_scales [rows_cap, K/128];
 * offsets: DEVICE int32[G+1], non-decreasing, offsets[0] = 0,
 *   offsets[G] <= rows_cap (precondition, not checked: it would need a
 *   synchronization); empty groups are allowed;
 * w: codes [G, N, K]; w_scales [G, ceil(N/128), K/128];
 * c: [rows_cap, ld_c] in grouped (expert-sorted) row order; rows not
 * covered by any group are not written.  out_dtype as for fp8q_gemm; the
 * partials are formed at float32 grade.
 * The kernel clamps every group's row range to [0, rows_cap] (a routing table
 * that breaks the precondition gives wrong rows for the groups it breaks,
 * never an access outside a or c). */
fp8q_status fp8q_grouped_gemm(const uint8_t* a, const float* a_scales,
                              const int32_t* offsets, int32_t G, int64_t rows_cap,
                              const uint8_t* w, const float* w_scales,
                              int64_t N, int64_t K, int out_dtype,
                              void* c, int64_t ld_c, hipStream_t stream);

/* fp8q_grouped_gemm with the accumulation form acc (FP8Q_ACC_*), as
 * fp8q_gemm_ex extends fp8q_gemm. */
fp8q_status fp8q_grouped_gemm_ex(const uint8_t* a, const float* a_scales,
                                 const int32_t* offsets, int32_t G, int64_t rows_cap,
                                 const uint8_t* w, const float* w_scales,
                                 int64_t N, int64_t K, int out_dtype, int acc,
                                 void* c, int64_t ld_c, hipStream_t stream);

/* FP8 weight gradient dW[Nout, Kin] = dY^T . X over T tokens
 * (jp-study.kr doc 258368 ¶3):
 *   dW[n,c] = sum_b dy_scales[n,b] * x_scales[c,b] * sum_{t in block b} dY[t,n] * X[t,c]
 * Operands are FP8Q_TILE_TOKEN_T outputs with ld_codes = T: dy_t codes
 * [Nout, T], dy_scales [Nout, T/128], x_t codes [Kin, T], x_scales
 * [Kin, T/128].  T must be a multiple of 128 (T = 0 writes zeros).  Partials
 * at float32 grade.  Output float32, row stride ld_dw elements, overwritten. */
fp8q_status fp8q_wgrad(const uint8_t* dy_t, const float* dy_scales,
                       const uint8_t* x_t, const float* x_scales,
                       int64_t Nout, int64_t Kin, int64_t T,
                       float* dw, int64_t ld_dw, hipStream_t stream);

/* fp8q_wgrad with the accumulation form acc (FP8Q_ACC_*), as fp8q_gemm_ex
 * extends fp8q_gemm. */
fp8q_status fp8q_wgrad_ex(const uint8_t* dy_t, const float* dy_scales,
                          const uint8_t* x_t, const float* x_scales,
                          int64_t Nout, int64_t Kin, int64_t T, int acc,
                          float* dw, int64_t ld_dw, hipStream_t stream);

/* FP8 dispatch gather (jp-study.kr doc 258368 ¶1: activations are quantized
 * once, before the MoE dispatch, and the FP8 codes travel instead of BF16).
 * Row i of the output is row index[i] of the quantized activation, codes and
 * 1x128 scales alike:
 *   out_codes[i, 0:cols]  = codes[index[i], 0:cols]
 *   out_scales[i, 0:nb]   = scales[index[i], 0:nb],  nb = ceil(cols/128)
 * codes [rows, ld_codes >= cols]; scales [rows, nb] (fp8q_quantize_act
 * output); index: DEVICE int32[n_out] (e.g. the expert-sorted token list of
 * one device; a token may appear several times).  An index outside
 * [0, rows) is not checked on the host (that would need a synchronization):
 * its output row is written as zero codes and a zero scale.  out_codes
 * [n_out, ld_out >= cols], out_scales [n_out, nb].  n_out <= 2^26 - 4 (one
 * wave per output row, four per workgroup, fewer than 2^24 workgroups), else
 * FP8Q_ERR_SHAPE. */
fp8q_status fp8q_gather_rows(const uint8_t* codes, int64_t rows, int64_t cols, int64_t ld_codes,
                             const float* scales, const int32_t* index, int64_t n_out,
                             uint8_t* out_codes, int64_t ld_out, float* out_scales,
                             hipStream_t stream);

/* SwiGLU of the MoE up-projection output, quantized for the down-projection
 * (tmdrlife.com wr_id=13334 ¶3-¶4: the SwiGLU operator of the MoE sits
 * between the two FP8 expert GEMMs; its inputs are cached in FP8 with
 * power-of-two scales and its output is recomputed from them in the
 * backward pass).  x: BF16 [rows, ld_x >= 2*inter], gate = x[:, 0:inter],
 * up = x[:, inter:2*inter].  Per element, in float32:
 *   y = bf16_rne( (g / (1 + exp(-g))) * u )
 * (the BF16 value an unfused SwiGLU would store), then y is quantized per
 * 1x128 tile along inter exactly as fp8q_quantize_act(FP8Q_TILE_ROW,
 * scale_mode) would quantize that BF16 tensor: codes [rows, ld_codes >=
 * inter], scales [rows, ceil(inter/128)].  exp is float32 with an error of
 * a few ulp, so y can differ from the correctly rounded BF16 of the exact
 * value when that value lies within a few float32 ulp of a rounding
 * boundary between two BF16 numbers.
 * Optional cache of the input: when cache_codes is not NULL (then
 * cache_scales must not be NULL either and inter must be a multiple of 128),
 * x itself is also quantized per 1x128 tile with cache_scale_mode (the
 * pages' choice is FP8Q_SCALE_POW2): cache_codes [rows, ld_cache >= 2*inter],
 * cache_scales [rows, 2*inter/128] -- bit for bit what fp8q_quantize_act
 * writes for x, from the same single read of x.  Inputs must be finite and
 * every y must be below the largest finite BF16 value. */
fp8q_status fp8q_swiglu_quantize(const void* x_bf16, int64_t rows, int64_t inter, int64_t ld_x,
                                 int scale_mode, uint8_t* codes, int64_t ld_codes, float* scales,
                                 int cache_scale_mode, uint8_t* cache_codes, int64_t ld_cache,
                                 float* cache_scales, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* fp8q_status_string(fp8q_status s);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
