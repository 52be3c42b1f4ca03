// C-ABI entry points of libfp8q.so: argument validation, device check and
// dispatch to the gfx950 kernels.  Every check runs before anything touches
// the GPU, so an argument error leaves the outputs untouched and launches
// nothing.
#include <atomic>
#include <cstring>

#include "fp8q.h"
#include "fp8q_internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxGroups = int64_t(1) << 24;  // 256-thread workgroups per launch
// 128x128 weight blocks per launch (one workgroup each; with the activation
// part of fp8q_quantize_linear, at most 2^20 more, still below kMaxGroups)
constexpr int64_t kMaxWeightBlocks = int64_t(1) << 23;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dim_ok(int64_t v) { return v >= 0 && v <= kMaxDim; }

// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

fp8q_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8Q_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int cached = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (cached) return cached == 1 ? FP8Q_OK : FP8Q_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8Q_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP8Q_OK : FP8Q_ERR_DEVICE;
}

fp8q_status launched(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* fp8q_status_string(fp8q_status s) {
  switch (s) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or unknown enum)";
    case FP8Q_ERR_SHAPE: return "bad shape (leading dimension too small, K not a multiple of 128, or size >= 2^31)";
    case FP8Q_ERR_ALIGN: return "misaligned base pointer (16-byte alignment required)";
    case FP8Q_ERR_LAUNCH: return "kernel launch failed";
    case FP8Q_ERR_DEVICE: return "current device is not an MI355X (gfx950)";
  }
  return "unknown status";
}

fp8q_status fp8q_quantize_act(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int tile_axis, int scale_mode, uint8_t* codes, int64_t ld_codes,
                              float* scales, hipStream_t stream) {
  if (!dim_ok(rows) || !dim_ok(cols) || !dim_ok(ld_x) || !dim_ok(ld_codes)) return FP8Q_ERR_INVALID_ARG;
  if (tile_axis != FP8Q_TILE_ROW && tile_axis != FP8Q_TILE_TOKEN_T) return FP8Q_ERR_INVALID_ARG;
  if (scale_mode != FP8Q_SCALE_FREE && scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8Q_OK;
  if (!x_bf16 || !codes || !scales) return FP8Q_ERR_INVALID_ARG;
  if (ld_x < cols) return FP8Q_ERR_SHAPE;
  const int64_t code_row = tile_axis == FP8Q_TILE_ROW ? cols : rows;
  if (ld_codes < code_row) return FP8Q_ERR_SHAPE;
  const int64_t tiles = tile_axis == FP8Q_TILE_ROW ? rows * ((cols + 127) / 128) : cols * ((rows + 127) / 128);
  if (tiles > kMaxDim) return FP8Q_ERR_SHAPE;
  // a launch's work items (256 per workgroup) must fit in 32 bits
  if (tile_axis == FP8Q_TILE_TOKEN_T && ((rows + 127) / 128) * ((cols + 63) / 64) >= kMaxGroups)
    return FP8Q_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales)) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  const bool pow2 = scale_mode == FP8Q_SCALE_POW2;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  if (tile_axis == FP8Q_TILE_ROW)
    return launched(fp8q::launch_quant_rows(x, (int)rows, (int)cols, ld_x, pow2, codes, ld_codes, scales, stream));
  return launched(fp8q::launch_quant_token_t(x, (int)rows, (int)cols, ld_x, pow2, codes, ld_codes, scales, stream));
}

fp8q_status fp8q_quantize_weight(const void* w_bf16, int64_t N, int64_t K, int64_t ld_w, int scale_mode,
                                 uint8_t* codes, int64_t ld_codes, float* scales, hipStream_t stream) {
  if (!dim_ok(N) || !dim_ok(K) || !dim_ok(ld_w) || !dim_ok(ld_codes)) return FP8Q_ERR_INVALID_ARG;
  if (scale_mode != FP8Q_SCALE_FREE && scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (!w_bf16 || !codes || !scales) return FP8Q_ERR_INVALID_ARG;
  if (ld_w < K || ld_codes < K) return FP8Q_ERR_SHAPE;
  if (((N + 127) / 128) * ((K + 127) / 128) >= kMaxWeightBlocks) return FP8Q_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(codes) || !aligned16(scales)) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_quant_blocks(static_cast<const uint16_t*>(w_bf16), (int)N, (int)K, ld_w,
                                            scale_mode == FP8Q_SCALE_POW2, codes, ld_codes, scales, stream));
}

fp8q_status fp8q_quantize_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ld_x, int act_scale_mode,
                                 uint8_t* a_codes, int64_t ld_a, float* a_scales, const void* w_bf16, int64_t N,
                                 int64_t ld_w, int weight_scale_mode, uint8_t* w_codes, int64_t ld_wc,
                                 float* w_scales, hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(K) || !dim_ok(N) || !dim_ok(ld_x) || !dim_ok(ld_a) || !dim_ok(ld_w) || !dim_ok(ld_wc))
    return FP8Q_ERR_INVALID_ARG;
  if (act_scale_mode != FP8Q_SCALE_FREE && act_scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  if (weight_scale_mode != FP8Q_SCALE_FREE && weight_scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  if (K == 0 || (M == 0 && N == 0)) return FP8Q_OK;
  if (M > 0 && (!x_bf16 || !a_codes || !a_scales)) return FP8Q_ERR_INVALID_ARG;
  if (N > 0 && (!w_bf16 || !w_codes || !w_scales)) return FP8Q_ERR_INVALID_ARG;
  if ((M > 0 && (ld_x < K || ld_a < K)) || (N > 0 && (ld_w < K || ld_wc < K))) return FP8Q_ERR_SHAPE;
  const int64_t nb = (K + 127) / 128;
  if (M * nb > kMaxDim || ((N + 127) / 128) * nb >= kMaxWeightBlocks) return FP8Q_ERR_SHAPE;
  if (M > 0 && (!aligned16(x_bf16) || !aligned16(a_codes) || !aligned16(a_scales))) return FP8Q_ERR_ALIGN;
  if (N > 0 && (!aligned16(w_bf16) || !aligned16(w_codes) || !aligned16(w_scales))) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_quant_linear(static_cast<const uint16_t*>(x_bf16), (int)M, (int)K, ld_x,
                                            act_scale_mode == FP8Q_SCALE_POW2, a_codes, ld_a, a_scales,
                                            static_cast<const uint16_t*>(w_bf16), (int)N, ld_w,
                                            weight_scale_mode == FP8Q_SCALE_POW2, w_codes, ld_wc, w_scales, stream));
}

fp8q_status fp8q_quantize_weight_t(const void* w_bf16, int64_t N, int64_t K, int64_t ld_w, int scale_mode,
                                   uint8_t* codes, int64_t ld_codes, float* scales,
                                   uint8_t* codes_t, int64_t ld_codes_t, float* scales_t, hipStream_t stream) {
  if (!dim_ok(N) || !dim_ok(K) || !dim_ok(ld_w) || !dim_ok(ld_codes) || !dim_ok(ld_codes_t))
    return FP8Q_ERR_INVALID_ARG;
  if (scale_mode != FP8Q_SCALE_FREE && scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return FP8Q_OK;
  if (!w_bf16 || !codes_t || !scales_t || (codes && !scales)) return FP8Q_ERR_INVALID_ARG;
  if (ld_w < K || ld_codes_t < N || (codes && ld_codes < K)) return FP8Q_ERR_SHAPE;
  if (((N + 127) / 128) * ((K + 127) / 128) >= kMaxWeightBlocks) return FP8Q_ERR_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(codes_t) || !aligned16(scales_t)) return FP8Q_ERR_ALIGN;
  if (codes && (!aligned16(codes) || !aligned16(scales))) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_quant_blocks_t(static_cast<const uint16_t*>(w_bf16), (int)N, (int)K, ld_w,
                                              scale_mode == FP8Q_SCALE_POW2, codes, ld_codes, scales, codes_t,
                                              ld_codes_t, scales_t, stream));
}

namespace {
// GEMM kernels address an operand with 32-bit byte offsets.
bool acc_ok(int acc) {
  return acc == FP8Q_ACC_FP32 || acc == FP8Q_ACC_FP8_MFMA || acc == FP8Q_ACC_FP8_MFMA_SCALED ||
         acc == FP8Q_ACC_FP32_POW2;
}

constexpr int64_t kMaxOperandBytes = int64_t(1) << 31;
// 512-thread GEMM workgroups per launch (work items must fit in 32 bits)
constexpr int64_t kMaxGemmTiles = int64_t(1) << 23;
int64_t tiles256(int64_t rows, int64_t cols, int64_t width) { return ((rows + 255) / 256) * ((cols + width - 1) / width); }

fp8q_status check_gemm_common(int64_t K, int out_dtype, const void* c, int64_t ld_c, int64_t N) {
  if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16) return FP8Q_ERR_INVALID_ARG;
  if (K % 128) return FP8Q_ERR_SHAPE;
  if (!c) return FP8Q_ERR_INVALID_ARG;
  if (ld_c < N) return FP8Q_ERR_SHAPE;
  if (!aligned16(c)) return FP8Q_ERR_ALIGN;
  return FP8Q_OK;
}
}  // namespace

fp8q_status fp8q_gemm_ex(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales,
                         int64_t M, int64_t N, int64_t K, int out_dtype, int acc, void* c, int64_t ld_c,
                         hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || !dim_ok(ld_c)) return FP8Q_ERR_INVALID_ARG;
  if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16) return FP8Q_ERR_INVALID_ARG;
  if (!acc_ok(acc)) return FP8Q_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8Q_OK;
  if (fp8q_status st = check_gemm_common(K, out_dtype, c, ld_c, N)) return st;
  // tiles of 224 or 256 columns: bound the count with the narrower width
  if (M * K >= kMaxOperandBytes || N * K >= kMaxOperandBytes || tiles256(M, N, 224) >= kMaxGemmTiles)
    return FP8Q_ERR_SHAPE;
  if (K > 0) {
    if (!a || !a_scales || !w || !w_scales) return FP8Q_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(w) || !aligned16(a_scales) || !aligned16(w_scales)) return FP8Q_ERR_ALIGN;
  }
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_gemm(a, a_scales, w, w_scales, (int)M, (int)N, (int)K,
                                    out_dtype == FP8Q_OUT_BF16, acc, c, ld_c, stream));
}

int64_t fp8q_set_gemm_small_limit(int64_t max_outputs) { return fp8q::set_small_gemm_limit(max_outputs); }

fp8q_status fp8q_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales,
                      int64_t M, int64_t N, int64_t K, int out_dtype, void* c, int64_t ld_c, hipStream_t stream) {
  return fp8q_gemm_ex(a, a_scales, w, w_scales, M, N, K, out_dtype, FP8Q_ACC_FP32, c, ld_c, stream);
}

fp8q_status fp8q_gemm_quantized(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales,
                                int64_t M, int64_t N, int64_t K, int acc, int scale_mode, uint8_t* c_codes,
                                int64_t ld_c, float* c_scales, hipStream_t stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || !dim_ok(ld_c)) return FP8Q_ERR_INVALID_ARG;
  if (!acc_ok(acc)) return FP8Q_ERR_INVALID_ARG;
  if (scale_mode != FP8Q_SCALE_FREE && scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP8Q_OK;
  if (!c_codes || !c_scales) return FP8Q_ERR_INVALID_ARG;
  if (K % 128) return FP8Q_ERR_SHAPE;
  if (ld_c < N) return FP8Q_ERR_SHAPE;
  if (M * K >= kMaxOperandBytes || N * K >= kMaxOperandBytes || M * ((N + 127) / 128) > kMaxDim ||
      tiles256(M, N, 256) >= kMaxGemmTiles)
    return FP8Q_ERR_SHAPE;
  if (!aligned16(c_codes) || !aligned16(c_scales)) return FP8Q_ERR_ALIGN;
  if (K > 0) {
    if (!a || !a_scales || !w || !w_scales) return FP8Q_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(w) || !aligned16(a_scales) || !aligned16(w_scales)) return FP8Q_ERR_ALIGN;
  }
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_gemm_quantized(a, a_scales, w, w_scales, (int)M, (int)N, (int)K, acc,
                                              scale_mode == FP8Q_SCALE_POW2, c_codes, ld_c, c_scales, stream));
}

fp8q_status fp8q_grouped_gemm_ex(const uint8_t* a, const float* a_scales, const int32_t* offsets, int32_t G,
                                 int64_t rows_cap, const uint8_t* w, const float* w_scales, int64_t N,
                                 int64_t K, int out_dtype, int acc, void* c, int64_t ld_c, hipStream_t stream) {
  if (G < 0 || !dim_ok(rows_cap) || !dim_ok(N) || !dim_ok(K) || !dim_ok(ld_c)) return FP8Q_ERR_INVALID_ARG;
  if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16) return FP8Q_ERR_INVALID_ARG;
  if (!acc_ok(acc)) return FP8Q_ERR_INVALID_ARG;
  if (G == 0 || rows_cap == 0 || N == 0) return FP8Q_OK;
  if (!offsets) return FP8Q_ERR_INVALID_ARG;
  if (fp8q_status st = check_gemm_common(K, out_dtype, c, ld_c, N)) return st;
  const int64_t tiles = ((rows_cap + 255) / 256 + G) * ((N + 255) / 256);
  if (tiles >= kMaxGemmTiles || rows_cap * K >= kMaxOperandBytes || int64_t(G) * N * K >= kMaxOperandBytes)
    return FP8Q_ERR_SHAPE;
  if (K > 0) {
    if (!a || !a_scales || !w || !w_scales) return FP8Q_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(w) || !aligned16(a_scales) || !aligned16(w_scales)) return FP8Q_ERR_ALIGN;
  }
  if (!aligned16(offsets)) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_grouped_gemm(a, a_scales, offsets, (int)G, (int)rows_cap, w, w_scales, (int)N,
                                            (int)K, out_dtype == FP8Q_OUT_BF16, acc, c,
                                            ld_c, stream));
}

fp8q_status fp8q_grouped_gemm(const uint8_t* a, const float* a_scales, const int32_t* offsets, int32_t G,
                              int64_t rows_cap, const uint8_t* w, const float* w_scales, int64_t N, int64_t K,
                              int out_dtype, void* c, int64_t ld_c, hipStream_t stream) {
  return fp8q_grouped_gemm_ex(a, a_scales, offsets, G, rows_cap, w, w_scales, N, K, out_dtype, FP8Q_ACC_FP32, c,
                              ld_c, stream);
}

fp8q_status fp8q_wgrad_ex(const uint8_t* dy_t, const float* dy_scales, const uint8_t* x_t, const float* x_scales,
                          int64_t Nout, int64_t Kin, int64_t T, int acc, float* dw, int64_t ld_dw,
                          hipStream_t stream) {
  if (!dim_ok(Nout) || !dim_ok(Kin) || !dim_ok(T) || !dim_ok(ld_dw)) return FP8Q_ERR_INVALID_ARG;
  if (!acc_ok(acc)) return FP8Q_ERR_INVALID_ARG;
  if (Nout == 0 || Kin == 0) return FP8Q_OK;
  if (fp8q_status st = check_gemm_common(T, FP8Q_OUT_F32, dw, ld_dw, Kin)) return st;
  // tiles of 224 or 256 columns: bound the count with the narrower width
  if (Nout * T >= kMaxOperandBytes || Kin * T >= kMaxOperandBytes || tiles256(Nout, Kin, 224) >= kMaxGemmTiles)
    return FP8Q_ERR_SHAPE;
  if (T > 0) {
    if (!dy_t || !dy_scales || !x_t || !x_scales) return FP8Q_ERR_INVALID_ARG;
    if (!aligned16(dy_t) || !aligned16(x_t) || !aligned16(dy_scales) || !aligned16(x_scales)) return FP8Q_ERR_ALIGN;
  }
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_wgrad(dy_t, dy_scales, x_t, x_scales, (int)Nout, (int)Kin, (int)T,
                                     acc, dw, ld_dw, stream));
}

fp8q_status fp8q_wgrad(const uint8_t* dy_t, const float* dy_scales, const uint8_t* x_t, const float* x_scales,
                       int64_t Nout, int64_t Kin, int64_t T, float* dw, int64_t ld_dw, hipStream_t stream) {
  return fp8q_wgrad_ex(dy_t, dy_scales, x_t, x_scales, Nout, Kin, T, FP8Q_ACC_FP32, dw, ld_dw, stream);
}

fp8q_status fp8q_gather_rows(const uint8_t* codes, int64_t rows, int64_t cols, int64_t ld_codes,
                             const float* scales, const int32_t* index, int64_t n_out, uint8_t* out_codes,
                             int64_t ld_out, float* out_scales, hipStream_t stream) {
  if (!dim_ok(rows) || !dim_ok(cols) || !dim_ok(ld_codes) || !dim_ok(n_out) || !dim_ok(ld_out))
    return FP8Q_ERR_INVALID_ARG;
  if (n_out == 0 || cols == 0) return FP8Q_OK;
  if (!index || !out_codes || !out_scales) return FP8Q_ERR_INVALID_ARG;
  if (rows > 0 && (!codes || !scales)) return FP8Q_ERR_INVALID_ARG;
  if (ld_codes < cols || ld_out < cols) return FP8Q_ERR_SHAPE;
  if (rows * ld_codes >= kMaxOperandBytes || n_out * ld_out >= kMaxOperandBytes) return FP8Q_ERR_SHAPE;
  if ((n_out + 3) / 4 >= kMaxGroups) return FP8Q_ERR_SHAPE;  // one wave per output row
  if (!aligned16(index) || !aligned16(out_codes) || !aligned16(out_scales)) return FP8Q_ERR_ALIGN;
  if (rows > 0 && (!aligned16(codes) || !aligned16(scales))) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_gather_rows(codes, (int)rows, (int)cols, ld_codes, scales, index, (int)n_out,
                                           out_codes, ld_out, out_scales, stream));
}

fp8q_status fp8q_swiglu_quantize(const void* x_bf16, int64_t rows, int64_t inter, int64_t ld_x, int scale_mode,
                                 uint8_t* codes, int64_t ld_codes, float* scales, int cache_scale_mode,
                                 uint8_t* cache_codes, int64_t ld_cache, float* cache_scales,
                                 hipStream_t stream) {
  if (!dim_ok(rows) || !dim_ok(inter) || !dim_ok(ld_x) || !dim_ok(ld_codes) || !dim_ok(ld_cache))
    return FP8Q_ERR_INVALID_ARG;
  if (scale_mode != FP8Q_SCALE_FREE && scale_mode != FP8Q_SCALE_POW2) return FP8Q_ERR_INVALID_ARG;
  const bool cache = cache_codes != nullptr;
  if (cache && cache_scale_mode != FP8Q_SCALE_FREE && cache_scale_mode != FP8Q_SCALE_POW2)
    return FP8Q_ERR_INVALID_ARG;
  if (rows == 0 || inter == 0) return FP8Q_OK;
  if (!x_bf16 || !codes || !scales || (cache && !cache_scales)) return FP8Q_ERR_INVALID_ARG;
  if (ld_x < 2 * inter || ld_codes < inter || (cache && ld_cache < 2 * inter)) return FP8Q_ERR_SHAPE;
  if (cache && inter % 128) return FP8Q_ERR_SHAPE;
  if (rows * ((inter + 127) / 128) > kMaxDim) return FP8Q_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales)) return FP8Q_ERR_ALIGN;
  if (cache && (!aligned16(cache_codes) || !aligned16(cache_scales))) return FP8Q_ERR_ALIGN;
  if (fp8q_status st = check_device()) return st;
  return launched(fp8q::launch_swiglu_quant(static_cast<const uint16_t*>(x_bf16), (int)rows, (int)inter, ld_x,
                                            scale_mode == FP8Q_SCALE_POW2, codes, ld_codes, scales,
                                            cache_scale_mode == FP8Q_SCALE_POW2, cache ? cache_codes : nullptr,
                                            ld_cache, cache ? cache_scales : nullptr, stream));
}

}  // extern "C"
