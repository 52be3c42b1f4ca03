// Internal declarations shared by the host entry points (fp8q_api.cpp) and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Grid sizes of the streaming kernels (host code; 64-bit arithmetic, so a
// tile count up to 2^31 - 1 cannot overflow here).
//  rows_grid: the 1x128 row quantizer, one pass per wave (16 tiles per
//    wave: 16 per 64-thread workgroup, 128 per 512-thread workgroup) up to
//    kMaxRowsGrid workgroups, then a grid-stride loop whose stride is
//    tiles_per_wg * kMaxRowsGrid tiles.
//  stream_grid: four waves per workgroup, up to kMaxStreamGrid workgroups.
constexpr int kMaxRowsGrid = 1 << 20;
constexpr int kMaxStreamGrid = 2048;
inline int rows_grid(int64_t ntiles, int tiles_per_wg = 64) {
  const int64_t want = (ntiles + tiles_per_wg - 1) / tiles_per_wg;
  return (int)(want < kMaxRowsGrid ? want : kMaxRowsGrid);
}
inline int stream_grid(int64_t waves_needed) {
  const int64_t wg = (waves_needed + 3) / 4;
  return (int)(wg < kMaxStreamGrid ? (wg > 0 ? wg : 1) : kMaxStreamGrid);
}

// Launchers validate nothing: fp8q_api.cpp has checked shapes, alignment and
// the device before calling them.  Every size here is > 0 and < 2^31.
hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, int64_t ldx, bool pow2,
                             uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream);
hipError_t launch_quant_token_t(const uint16_t* x, int rows, int cols, int64_t ldx, bool pow2,
                                uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream);
hipError_t launch_quant_blocks(const uint16_t* w, int n, int k, int64_t ldw, bool pow2,
                               uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream);

// the activation x [m, k] in 1x128 tiles and the weight w [n, k] in 128x128
// blocks, one launch
hipError_t launch_quant_linear(const uint16_t* x, int m, int k, int64_t ldx, bool a_pow2, uint8_t* a_codes,
                               int64_t lda, float* a_scales, const uint16_t* w, int n, int64_t ldw, bool w_pow2,
                               uint8_t* w_codes, int64_t ldwc, float* w_scales, hipStream_t stream);

hipError_t launch_quant_blocks_t(const uint16_t* w, int n, int k, int64_t ldw, bool pow2,
                                 uint8_t* codes, int64_t ldc, float* scales, uint8_t* codes_t,
                                 int64_t ldt, float* scales_t, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                       const float* w_scales, int m, int n, int k, bool bf16_out, int acc,
                       void* c, int64_t ldc, hipStream_t stream);
// float32-grade dense GEMM over 32 x 32 output tiles with the K blocks split
// over four waves (gemm_small.hip); launch_gemm takes it for outputs of at
// most small_gemm_limit() elements
hipError_t launch_gemm_small(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales,
                             int m, int n, int k, bool bf16_out, void* c, int64_t ldc, hipStream_t stream);
// outputs (M * N) up to which the dense float32-grade GEMM uses the small
// kernel: the value set by set_small_gemm_limit, or, while none is set (or
// after a negative one), 8192 per compute unit of the current device
int64_t small_gemm_limit();
int64_t set_small_gemm_limit(int64_t max_outputs);  // returns the previous setting (-1: the default)
int device_cus();
// C = A . W^T rounded to BF16, quantized per 1x128 tile along N
hipError_t launch_gemm_quantized(const uint8_t* a, const float* a_scales, const uint8_t* w,
                                 const float* w_scales, int m, int n, int k, int acc, bool pow2,
                                 uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream);
hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_scales, const int32_t* offsets,
                               int groups, int rows_cap, const uint8_t* w, const float* w_scales,
                               int n, int k, bool bf16_out, int acc, void* c, int64_t ldc,
                               hipStream_t stream);
hipError_t launch_wgrad(const uint8_t* dy_t, const float* dy_scales, const uint8_t* x_t,
                        const float* x_scales, int nout, int kin, int t, int acc, float* dw,
                        int64_t lddw, hipStream_t stream);

hipError_t launch_gather_rows(const uint8_t* codes, int rows, int cols, int64_t ldc, const float* scales,
                              const int32_t* index, int n_out, uint8_t* out, int64_t ldo, float* out_scales,
                              hipStream_t stream);
// ccodes == nullptr: no cache of the input (cache_pow2, ldcc, cscales unused)
hipError_t launch_swiglu_quant(const uint16_t* x, int rows, int inter, int64_t ldx, bool pow2, uint8_t* codes,
                               int64_t ldc, float* scales, bool cache_pow2, uint8_t* ccodes, int64_t ldcc,
                               float* cscales, hipStream_t stream);

}  // namespace fp8q
