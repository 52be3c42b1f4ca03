// Host-side check of the C ABI's entry points (fp8q_api.cpp), built for the
// CPU with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_abi_host_sanitized.py.  The kernel launchers and the two HIP
// runtime calls the entry points make (hipGetDevice, hipGetDeviceProperties)
// are replaced by stubs, so every path runs without a GPU: argument errors,
// the device check and its per-device cache, the hand-over of each argument
// to its launcher, and the mapping of a failed launch to FP8Q_ERR_LAUNCH.
// Prints "host ABI checks passed" and returns 0 when every check holds.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "fp8q.h"
#include "fp8q_internal.h"

namespace {

int g_failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::printf("%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                      \
    }                                                                    \
  } while (0)

// ---- fake device: id g_dev (negative: no device); id 1 reports gfx942,
// id 2 a gfx950 with target features, every other id plain gfx950
int g_dev = 0;
int g_prop_queries = 0;

// ---- launcher stubs: the last call's name and arguments
struct Call {
  std::string name;
  std::vector<int64_t> ints;
  std::vector<const void*> ptrs;
  hipStream_t stream = nullptr;
};
Call g_last;
int g_calls = 0;
hipError_t g_launch_result = hipSuccess;

hipError_t record(const char* name, std::vector<int64_t> ints, std::vector<const void*> ptrs, hipStream_t s) {
  g_last.name = name;
  g_last.ints = std::move(ints);
  g_last.ptrs = std::move(ptrs);
  g_last.stream = s;
  ++g_calls;
  return g_launch_result;
}

}  // namespace

extern "C" hipError_t hipGetDevice(int* device) {
  if (g_dev < 0) return hipErrorNoDevice;
  *device = g_dev;
  return hipSuccess;
}

extern "C" hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int device) {
  ++g_prop_queries;
  std::memset(prop, 0, sizeof(*prop));
  const char* arch = device == 1 ? "gfx942" : device == 2 ? "gfx950:sramecc+:xnack-" : "gfx950";
  std::strncpy(prop->gcnArchName, arch, sizeof(prop->gcnArchName) - 1);
  return hipSuccess;
}

namespace fp8q {

hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, int64_t ldx, bool pow2, uint8_t* codes,
                             int64_t ldc, float* scales, hipStream_t s) {
  return record("quant_rows", {rows, cols, ldx, pow2, ldc}, {x, codes, scales}, s);
}
hipError_t launch_quant_token_t(const uint16_t* x, int rows, int cols, int64_t ldx, bool pow2, uint8_t* codes,
                                int64_t ldc, float* scales, hipStream_t s) {
  return record("quant_token_t", {rows, cols, ldx, pow2, ldc}, {x, codes, scales}, s);
}
hipError_t launch_quant_blocks(const uint16_t* w, int n, int k, int64_t ldw, bool pow2, uint8_t* codes,
                               int64_t ldc, float* scales, hipStream_t s) {
  return record("quant_blocks", {n, k, ldw, pow2, ldc}, {w, codes, scales}, s);
}
hipError_t launch_quant_linear(const uint16_t* x, int m, int k, int64_t ldx, bool a_pow2, uint8_t* a_codes,
                               int64_t lda, float* a_scales, const uint16_t* w, int n, int64_t ldw, bool w_pow2,
                               uint8_t* w_codes, int64_t ldwc, float* w_scales, hipStream_t s) {
  return record("quant_linear", {m, k, ldx, a_pow2, lda, n, ldw, w_pow2, ldwc},
                {x, a_codes, a_scales, w, w_codes, w_scales}, s);
}
hipError_t launch_quant_blocks_t(const uint16_t* w, int n, int k, int64_t ldw, bool pow2, uint8_t* codes,
                                 int64_t ldc, float* scales, uint8_t* codes_t, int64_t ldt, float* scales_t,
                                 hipStream_t s) {
  return record("quant_blocks_t", {n, k, ldw, pow2, ldc, ldt}, {w, codes, scales, codes_t, scales_t}, s);
}
hipError_t launch_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales, int m,
                       int n, int k, bool bf16_out, int acc, void* c, int64_t ldc, hipStream_t s) {
  return record("gemm", {m, n, k, bf16_out, acc, ldc}, {a, a_scales, w, w_scales, c}, s);
}
hipError_t launch_gemm_quantized(const uint8_t* a, const float* a_scales, const uint8_t* w,
                                 const float* w_scales, int m, int n, int k, int acc, bool pow2, uint8_t* codes,
                                 int64_t ldc, float* scales, hipStream_t s) {
  return record("gemm_quantized", {m, n, k, acc, pow2, ldc}, {a, a_scales, w, w_scales, codes, scales}, s);
}
hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_scales, const int32_t* offsets, int groups,
                               int rows_cap, const uint8_t* w, const float* w_scales, int n, int k, bool bf16_out,
                               int acc, void* c, int64_t ldc, hipStream_t s) {
  return record("grouped_gemm", {groups, rows_cap, n, k, bf16_out, acc, ldc}, {a, a_scales, offsets, w, w_scales, c},
                s);
}
hipError_t launch_wgrad(const uint8_t* dy_t, const float* dy_scales, const uint8_t* x_t, const float* x_scales,
                        int nout, int kin, int t, int acc, float* dw, int64_t lddw, hipStream_t s) {
  return record("wgrad", {nout, kin, t, acc, lddw}, {dy_t, dy_scales, x_t, x_scales, dw}, s);
}
hipError_t launch_gather_rows(const uint8_t* codes, int rows, int cols, int64_t ldc, const float* scales,
                              const int32_t* index, int n_out, uint8_t* out, int64_t ldo, float* out_scales,
                              hipStream_t s) {
  return record("gather_rows", {rows, cols, ldc, n_out, ldo}, {codes, scales, index, out, out_scales}, s);
}
hipError_t launch_swiglu_quant(const uint16_t* x, int rows, int inter, int64_t ldx, bool pow2, uint8_t* codes,
                               int64_t ldc, float* scales, bool cache_pow2, uint8_t* ccodes, int64_t ldcc,
                               float* cscales, hipStream_t s) {
  return record("swiglu_quant", {rows, inter, ldx, pow2, ldc, cache_pow2, ldcc},
                {x, codes, scales, ccodes, cscales}, s);
}
int64_t g_small_limit_stub = -1;
int64_t set_small_gemm_limit(int64_t max_outputs) {
  const int64_t prev = g_small_limit_stub;
  g_small_limit_stub = max_outputs < 0 ? -1 : max_outputs;
  return prev;
}

}  // namespace fp8q

namespace {

// distinct, 16-byte aligned addresses that are never dereferenced
template <class T>
T* addr(uintptr_t i) {
  return reinterpret_cast<T*>(uintptr_t(0x10000) + 0x100 * i);
}
template <class T>
T* odd(uintptr_t i) {
  return reinterpret_cast<T*>(uintptr_t(0x10000) + 0x100 * i + 8);
}
hipStream_t stream_tag() { return reinterpret_cast<hipStream_t>(uintptr_t(0xABC0)); }

// Runs `call` and checks its status and whether it reached a launcher.
template <class F>
void expect(F call, fp8q_status want, bool launches, int line) {
  const int before = g_calls;
  const fp8q_status got = call();
  if (got != want || (g_calls != before) != launches) {
    std::printf("line %d: status %d (want %d), launched %d (want %d)\n", line, (int)got, (int)want,
                g_calls != before, (int)launches);
    ++g_failures;
  }
}
#define EXPECT(call, want, launches) expect([&] { return call; }, want, launches, __LINE__)

bool last_is(const char* name, std::vector<int64_t> ints, std::vector<const void*> ptrs) {
  return g_last.name == name && g_last.ints == ints && g_last.ptrs == ptrs && g_last.stream == stream_tag();
}

void device_check() {
  const auto* a = addr<uint8_t>(1);
  const auto* sa = addr<float>(2);
  const auto* w = addr<uint8_t>(3);
  const auto* sw = addr<float>(4);
  void* c = addr<void>(5);
  auto gemm = [&] { return fp8q_gemm(a, sa, w, sw, 256, 256, 256, FP8Q_OUT_BF16, c, 256, stream_tag()); };
  g_dev = -1;
  EXPECT(gemm(), FP8Q_ERR_DEVICE, false);
  // another architecture: refused, and the answer is cached per device
  g_dev = 1;
  int q0 = g_prop_queries;
  EXPECT(gemm(), FP8Q_ERR_DEVICE, false);
  EXPECT(gemm(), FP8Q_ERR_DEVICE, false);
  CHECK(g_prop_queries == q0 + 1);
  // gfx950 with target features in the name
  g_dev = 2;
  EXPECT(gemm(), FP8Q_OK, true);
  // a device id past the cache is still checked, every time
  g_dev = 100;
  q0 = g_prop_queries;
  EXPECT(gemm(), FP8Q_OK, true);
  EXPECT(gemm(), FP8Q_OK, true);
  CHECK(g_prop_queries == q0 + 2);
  g_dev = 0;
  q0 = g_prop_queries;
  EXPECT(gemm(), FP8Q_OK, true);
  EXPECT(gemm(), FP8Q_OK, true);
  CHECK(g_prop_queries == q0 + 1);
  // a failed launch
  g_launch_result = hipErrorLaunchFailure;
  EXPECT(gemm(), FP8Q_ERR_LAUNCH, true);
  g_launch_result = hipSuccess;
}

void quantizers() {
  const void* x = addr<void>(1);
  auto* codes = addr<uint8_t>(2);
  auto* scales = addr<float>(3);
  EXPECT(fp8q_quantize_act(x, 300, 7168, 7200, FP8Q_TILE_ROW, FP8Q_SCALE_POW2, codes, 7184, scales, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("quant_rows", {300, 7168, 7200, 1, 7184}, {x, codes, scales}));
  EXPECT(fp8q_quantize_act(x, 300, 72, 80, FP8Q_TILE_TOKEN_T, FP8Q_SCALE_FREE, codes, 304, scales, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("quant_token_t", {300, 72, 80, 0, 304}, {x, codes, scales}));
  EXPECT(fp8q_quantize_act(x, 300, 72, 80, FP8Q_TILE_TOKEN_T, FP8Q_SCALE_FREE, codes, 299, scales, stream_tag()),
         FP8Q_ERR_SHAPE, false);
  // 2^31 tiles or more
  EXPECT(fp8q_quantize_act(x, 1 << 16, 1 << 24, 1 << 24, FP8Q_TILE_TOKEN_T, FP8Q_SCALE_FREE, codes, 1 << 16,
                           scales, stream_tag()),
         FP8Q_ERR_SHAPE, false);
  // 2^24 workgroups (128 token blocks x 2^17 feature groups): one too many
  EXPECT(fp8q_quantize_act(x, 1 << 14, 1 << 23, 1 << 23, FP8Q_TILE_TOKEN_T, FP8Q_SCALE_FREE, codes, 1 << 14,
                           scales, stream_tag()),
         FP8Q_ERR_SHAPE, false);
  // 4M features (65536 groups of 64) over 128 token blocks: 2^29 tiles
  EXPECT(fp8q_quantize_act(x, 1 << 14, 1 << 22, 1 << 22, FP8Q_TILE_TOKEN_T, FP8Q_SCALE_FREE, codes, 1 << 14,
                           scales, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("quant_token_t", {1 << 14, 1 << 22, 1 << 22, 0, 1 << 14}, {x, codes, scales}));
  EXPECT(fp8q_quantize_act(x, int64_t(1) << 31, 8, 8, FP8Q_TILE_ROW, FP8Q_SCALE_FREE, codes, 8, scales, stream_tag()),
         FP8Q_ERR_INVALID_ARG, false);
  EXPECT(fp8q_quantize_act(odd<void>(1), 4, 8, 8, FP8Q_TILE_ROW, FP8Q_SCALE_FREE, codes, 8, scales, stream_tag()),
         FP8Q_ERR_ALIGN, false);
  EXPECT(fp8q_quantize_act(nullptr, 0, 8, 8, FP8Q_TILE_ROW, FP8Q_SCALE_FREE, nullptr, 8, nullptr, stream_tag()),
         FP8Q_OK, false);

  EXPECT(fp8q_quantize_weight(x, 4096, 7168, 7168, FP8Q_SCALE_FREE, codes, 7168, scales, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("quant_blocks", {4096, 7168, 7168, 0, 7168}, {x, codes, scales}));
  EXPECT(fp8q_quantize_weight(x, 4096, 7168, 7168, 2, codes, 7168, scales, stream_tag()), FP8Q_ERR_INVALID_ARG,
         false);
  // 2^23 blocks of 128 x 128 (2^12 x 2^11 blocks): one workgroup each, too many
  EXPECT(fp8q_quantize_weight(x, int64_t(1) << 19, int64_t(1) << 18, int64_t(1) << 18, FP8Q_SCALE_FREE, codes,
                              int64_t(1) << 18, scales, stream_tag()),
         FP8Q_ERR_SHAPE, false);

  const void* w = addr<void>(4);
  auto* wc = addr<uint8_t>(5);
  auto* ws = addr<float>(6);
  EXPECT(fp8q_quantize_linear(x, 64, 256, 256, FP8Q_SCALE_POW2, codes, 256, scales, w, 200, 256, FP8Q_SCALE_FREE, wc,
                              256, ws, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("quant_linear", {64, 256, 256, 1, 256, 200, 256, 0, 256}, {x, codes, scales, w, wc, ws}));
  // only the weight (M = 0): the activation pointers may be null
  EXPECT(fp8q_quantize_linear(nullptr, 0, 256, 0, FP8Q_SCALE_FREE, nullptr, 0, nullptr, w, 200, 256,
                              FP8Q_SCALE_FREE, wc, 256, ws, stream_tag()),
         FP8Q_OK, true);
  EXPECT(fp8q_quantize_linear(x, 64, 256, 128, FP8Q_SCALE_FREE, codes, 256, scales, w, 200, 256, FP8Q_SCALE_FREE,
                              wc, 256, ws, stream_tag()),
         FP8Q_ERR_SHAPE, false);

  auto* ct = addr<uint8_t>(7);
  auto* st = addr<float>(8);
  EXPECT(fp8q_quantize_weight_t(x, 300, 256, 256, FP8Q_SCALE_FREE, nullptr, 0, nullptr, ct, 304, st, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("quant_blocks_t", {300, 256, 256, 0, 0, 304}, {x, nullptr, nullptr, ct, st}));
  EXPECT(fp8q_quantize_weight_t(x, 300, 256, 256, FP8Q_SCALE_FREE, codes, 256, nullptr, ct, 304, st, stream_tag()),
         FP8Q_ERR_INVALID_ARG, false);
}

void gemms() {
  const auto* a = addr<uint8_t>(1);
  const auto* sa = addr<float>(2);
  const auto* w = addr<uint8_t>(3);
  const auto* sw = addr<float>(4);
  void* c = addr<void>(5);
  // the plain entry point runs the float32-grade form
  EXPECT(fp8q_gemm(a, sa, w, sw, 4096, 4096, 7168, FP8Q_OUT_BF16, c, 4104, stream_tag()), FP8Q_OK, true);
  CHECK(last_is("gemm", {4096, 4096, 7168, 1, FP8Q_ACC_FP32, 4104}, {a, sa, w, sw, c}));
  EXPECT(fp8q_gemm_ex(a, sa, w, sw, 4096, 4096, 7168, FP8Q_OUT_BF16, FP8Q_ACC_FP8_MFMA, c, 4104, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("gemm", {4096, 4096, 7168, 1, FP8Q_ACC_FP8_MFMA, 4104}, {a, sa, w, sw, c}));
  EXPECT(fp8q_gemm_ex(a, sa, w, sw, 64, 32, 256, FP8Q_OUT_F32, FP8Q_ACC_FP8_MFMA_SCALED, c, 32, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("gemm", {64, 32, 256, 0, FP8Q_ACC_FP8_MFMA_SCALED, 32}, {a, sa, w, sw, c}));
  EXPECT(fp8q_gemm(a, sa, w, sw, 4, 4, 100, FP8Q_OUT_F32, c, 4, stream_tag()), FP8Q_ERR_SHAPE, false);
  EXPECT(fp8q_gemm_ex(a, sa, w, sw, 4, 4, 100, FP8Q_OUT_F32, FP8Q_ACC_FP32, c, 4, stream_tag()), FP8Q_ERR_SHAPE,
         false);
  EXPECT(fp8q_gemm_ex(a, sa, w, sw, 4, 4, 128, FP8Q_OUT_F32, 4, c, 4, stream_tag()), FP8Q_ERR_INVALID_ARG, false);
  EXPECT(fp8q_gemm_ex(a, sa, w, sw, 64, 32, 256, FP8Q_OUT_BF16, FP8Q_ACC_FP32_POW2, c, 32, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("gemm", {64, 32, 256, 1, FP8Q_ACC_FP32_POW2, 32}, {a, sa, w, sw, c}));
  EXPECT(fp8q_gemm(a, sa, w, sw, 4, 4, 128, 2, c, 4, stream_tag()), FP8Q_ERR_INVALID_ARG, false);
  // an operand of 2 GiB or more (32-bit byte offsets in the kernels)
  EXPECT(fp8q_gemm(a, sa, w, sw, 1 << 24, 4, 128, FP8Q_OUT_F32, c, 4, stream_tag()), FP8Q_ERR_SHAPE, false);
  // 2^23 tiles of 256 x 256 (2^12 x 2^11): too many workgroups for one launch
  EXPECT(fp8q_gemm(a, sa, w, sw, int64_t(1) << 20, int64_t(1) << 19, 0, FP8Q_OUT_F32, c, int64_t(1) << 19,
                   stream_tag()),
         FP8Q_ERR_SHAPE, false);
  // K = 0: C = 0 is written by the kernel, operand pointers may be null
  EXPECT(fp8q_gemm(nullptr, nullptr, nullptr, nullptr, 4, 4, 0, FP8Q_OUT_F32, c, 4, stream_tag()), FP8Q_OK, true);
  EXPECT(fp8q_gemm(a, sa, w, odd<float>(4), 4, 4, 128, FP8Q_OUT_F32, c, 4, stream_tag()), FP8Q_ERR_ALIGN, false);

  auto* cc = addr<uint8_t>(6);
  auto* cs = addr<float>(7);
  EXPECT(fp8q_gemm_quantized(a, sa, w, sw, 100, 384, 256, FP8Q_ACC_FP32, FP8Q_SCALE_POW2, cc, 384, cs, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("gemm_quantized", {100, 384, 256, FP8Q_ACC_FP32, 1, 384}, {a, sa, w, sw, cc, cs}));

  const auto* offs = addr<int32_t>(8);
  EXPECT(fp8q_grouped_gemm(a, sa, offs, 16, 8776, w, sw, 4096, 7168, FP8Q_OUT_BF16, c, 4096, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("grouped_gemm", {16, 8776, 4096, 7168, 1, FP8Q_ACC_FP32, 4096}, {a, sa, offs, w, sw, c}));
  EXPECT(fp8q_grouped_gemm_ex(a, sa, offs, 16, 8776, w, sw, 4096, 7168, FP8Q_OUT_F32, FP8Q_ACC_FP8_MFMA, c, 4096,
                              stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("grouped_gemm", {16, 8776, 4096, 7168, 0, FP8Q_ACC_FP8_MFMA, 4096}, {a, sa, offs, w, sw, c}));
  EXPECT(fp8q_grouped_gemm_ex(a, sa, offs, 16, 8776, w, sw, 4096, 7168, FP8Q_OUT_F32, 7, c, 4096, stream_tag()),
         FP8Q_ERR_INVALID_ARG, false);
  EXPECT(fp8q_grouped_gemm(a, sa, nullptr, 16, 8776, w, sw, 4096, 7168, FP8Q_OUT_BF16, c, 4096, stream_tag()),
         FP8Q_ERR_INVALID_ARG, false);
  EXPECT(fp8q_grouped_gemm(a, sa, offs, -1, 8776, w, sw, 4096, 7168, FP8Q_OUT_BF16, c, 4096, stream_tag()),
         FP8Q_ERR_INVALID_ARG, false);
  // G experts of N x K codes must stay below 2 GiB
  EXPECT(fp8q_grouped_gemm(a, sa, offs, 80, 8776, w, sw, 4096, 7168, FP8Q_OUT_BF16, c, 4096, stream_tag()),
         FP8Q_ERR_SHAPE, false);

  auto* dw = addr<float>(9);
  EXPECT(fp8q_wgrad(a, sa, w, sw, 2048, 7168, 16384, dw, 7168, stream_tag()), FP8Q_OK, true);
  CHECK(last_is("wgrad", {2048, 7168, 16384, FP8Q_ACC_FP32, 7168}, {a, sa, w, sw, dw}));
  EXPECT(fp8q_wgrad_ex(a, sa, w, sw, 2048, 7168, 16384, FP8Q_ACC_FP8_MFMA_SCALED, dw, 7168, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("wgrad", {2048, 7168, 16384, FP8Q_ACC_FP8_MFMA_SCALED, 7168}, {a, sa, w, sw, dw}));
  EXPECT(fp8q_wgrad_ex(a, sa, w, sw, 2048, 7168, 16384, -1, dw, 7168, stream_tag()), FP8Q_ERR_INVALID_ARG, false);
  EXPECT(fp8q_wgrad(a, sa, w, sw, 2048, 7168, 16100, dw, 7168, stream_tag()), FP8Q_ERR_SHAPE, false);
}

void moe_glue() {
  const auto* codes = addr<uint8_t>(1);
  const auto* scales = addr<float>(2);
  const auto* index = addr<int32_t>(3);
  auto* out = addr<uint8_t>(4);
  auto* out_s = addr<float>(5);
  EXPECT(fp8q_gather_rows(codes, 8192, 7168, 7168, scales, index, 3773, out, 7168, out_s, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("gather_rows", {8192, 7168, 7168, 3773, 7168}, {codes, scales, index, out, out_s}));
  EXPECT(fp8q_gather_rows(codes, 8192, 7168, 7168, scales, nullptr, 3773, out, 7168, out_s, stream_tag()),
         FP8Q_ERR_INVALID_ARG, false);
  // one wave per output row: 2^26 rows (of 16 codes) are too many for one launch
  EXPECT(fp8q_gather_rows(codes, 8192, 16, 16, scales, index, int64_t(1) << 26, out, 16, out_s, stream_tag()),
         FP8Q_ERR_SHAPE, false);
  EXPECT(fp8q_gather_rows(codes, 8192, 16, 16, scales, index, (int64_t(1) << 26) - 4, out, 16, out_s, stream_tag()),
         FP8Q_OK, true);

  const void* x = addr<void>(6);
  auto* ccodes = addr<uint8_t>(7);
  auto* cscales = addr<float>(8);
  EXPECT(fp8q_swiglu_quantize(x, 3773, 2048, 4096, FP8Q_SCALE_POW2, out, 2048, out_s, FP8Q_SCALE_POW2, ccodes, 4096,
                              cscales, stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("swiglu_quant", {3773, 2048, 4096, 1, 2048, 1, 4096}, {x, out, out_s, ccodes, cscales}));
  // no cache: its mode is not checked and its pointers are passed as null
  EXPECT(fp8q_swiglu_quantize(x, 3773, 2048, 4096, FP8Q_SCALE_FREE, out, 2048, out_s, 9, nullptr, 0, cscales,
                              stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("swiglu_quant", {3773, 2048, 4096, 0, 2048, 0, 0}, {x, out, out_s, nullptr, nullptr}));
  EXPECT(fp8q_swiglu_quantize(x, 3773, 2000, 4000, FP8Q_SCALE_FREE, out, 2048, out_s, FP8Q_SCALE_FREE, ccodes, 4096,
                              cscales, stream_tag()),
         FP8Q_ERR_SHAPE, false);
}

// The largest row counts the entry points accept reach the kernels' tile
// sweeps: a tile index plus one stride of the sweep must stay below 2^32 (the
// kernels count tiles in 32-bit unsigned), and the grid helpers must not
// overflow.
void large_sweeps() {
  const void* x = addr<void>(1);
  auto* codes = addr<uint8_t>(2);
  auto* scales = addr<float>(3);
  const int64_t rows = (int64_t(1) << 31) - (int64_t(1) << 25);
  EXPECT(fp8q_quantize_act(x, rows, 1, 16, FP8Q_TILE_ROW, FP8Q_SCALE_FREE, codes, 16, scales, stream_tag()), FP8Q_OK,
         true);
  CHECK(last_is("quant_rows", {rows, 1, 16, 0, 16}, {x, codes, scales}));
  EXPECT(fp8q_quantize_linear(x, rows, 1, 16, FP8Q_SCALE_POW2, codes, 16, scales, nullptr, 0, 16, FP8Q_SCALE_FREE,
                              nullptr, 16, nullptr, stream_tag()),
         FP8Q_OK, true);
  EXPECT(fp8q_swiglu_quantize(x, rows, 1, 2, FP8Q_SCALE_FREE, codes, 16, scales, FP8Q_SCALE_FREE, nullptr, 0, nullptr,
                              stream_tag()),
         FP8Q_OK, true);
  CHECK(last_is("swiglu_quant", {rows, 1, 2, 0, 16, 0, 0}, {x, codes, scales, nullptr, nullptr}));
  // one tile more than the 32-bit signed range is refused
  EXPECT(fp8q_quantize_act(x, int64_t(1) << 30, 257, 272, FP8Q_TILE_ROW, FP8Q_SCALE_FREE, codes, 272, scales,
                           stream_tag()),
         FP8Q_ERR_SHAPE, false);
  for (int64_t ntiles : {int64_t(1), int64_t(63), int64_t(64), int64_t(1) << 26, rows, (int64_t(1) << 31) - 1}) {
    for (int per_wg : {16, 128}) {  // one-wave and eight-wave workgroups
      const int g = fp8q::rows_grid(ntiles, per_wg);
      CHECK(g >= 1 && g <= fp8q::kMaxRowsGrid);
      CHECK(int64_t(g) * per_wg >= std::min<int64_t>(ntiles, int64_t(fp8q::kMaxRowsGrid) * per_wg));
      const uint64_t stride = uint64_t(g) * per_wg;  // tiles per sweep of the whole grid
      CHECK(uint64_t(ntiles - 1) + stride < (uint64_t(1) << 32));
    }
    const int sg = fp8q::stream_grid((ntiles + 3) / 4);
    CHECK(sg >= 1 && sg <= fp8q::kMaxStreamGrid);
    CHECK(uint64_t(ntiles - 1) + uint64_t(sg) * 16 < (uint64_t(1) << 32));
  }
}

void status_strings() {
  for (int s = FP8Q_OK; s <= FP8Q_ERR_DEVICE; ++s) CHECK(std::strlen(fp8q_status_string((fp8q_status)s)) > 0);
  CHECK(std::strcmp(fp8q_status_string((fp8q_status)42), "unknown status") == 0);
}

}  // namespace

// The tiling limit of the dense GEMM is handed to the library unchanged and
// the previous setting comes back (negative values mean the default, -1).
void small_gemm_limit() {
  CHECK(fp8q_set_gemm_small_limit(0) == -1);
  CHECK(fp8q_set_gemm_small_limit(int64_t(1) << 40) == 0);
  CHECK(fp8q_set_gemm_small_limit(-7) == (int64_t(1) << 40));
  CHECK(fp8q_set_gemm_small_limit(-1) == -1);
}

int main() {
  device_check();
  small_gemm_limit();
  quantizers();
  gemms();
  moe_glue();
  large_sweeps();
  status_strings();
  if (g_failures) {
    std::printf("%d host ABI checks failed\n", g_failures);
    return 1;
  }
  std::printf("host ABI checks passed (%d launcher calls)\n", g_calls);
  return 0;
}
