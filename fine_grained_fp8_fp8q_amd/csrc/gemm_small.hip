// Block-scaled FP8 (E4M3) GEMM for outputs too small to fill the compute
// units with 256-wide tiles (gfx950).
//
// Same product as the float32-grade form of gemm.hip (tmdrlife.com
// wr_id=13334 ¶3; jp-study.kr doc 258368 ¶3): per 128-element block of K,
// the E4M3 x E4M3 partial is formed exactly widened to BF16 on the BF16
// matrix core (v_mfma_f32_16x16x32_bf16, float32 accumulator) and folded
// into FP32 with the block's activation and weight scales.
//
// A 128 x 256 output over K = 512 is one 256 x 256 tile: one compute unit
// runs four K blocks back to back while 255 stay idle.  Here a workgroup owns
// a 32 x 32 output tile and its four waves split the K blocks (wave w takes
// blocks w, w + 4, ...), so that output spreads over 32 compute units and
// each wave runs one block.  A wave loads its operand bytes straight into
// registers (no LDS staging: no other wave reads them), the next block's
// while it multiplies the current one, and folds each block's partial into
// its own FP32 accumulators.  The four waves' sums are then added in LDS in
// a fixed order (wave 0 + 1 + 2 + 3), so the result does not depend on
// timing.
#include "fp8q_internal.h"
#include "quant_common.h"

namespace fp8q {
namespace {

typedef int sm_v4i __attribute__((ext_vector_type(4)));
typedef float sm_v4f __attribute__((ext_vector_type(4)));
typedef __bf16 sm_v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 sm_v8bf __attribute__((ext_vector_type(8)));

constexpr int kTile = 32;   // output rows and columns per workgroup
constexpr int kWaves = 4;   // K blocks are dealt round-robin over these
constexpr int kRsrcFlagsSmall = 0x00020000;  // raw buffer access

// Eight E4M3 codes (two dwords) -> eight BF16 values, exactly.
__device__ __forceinline__ sm_v8bf small_e4m3x8_to_bf16(int lo, int hi) {
  const sm_v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, false);
  const sm_v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, true);
  const sm_v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, false);
  const sm_v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, true);
  return sm_v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One K block's operands in registers: lane (row r16 of a 16-row fragment,
// lane group g) holds bytes 32g..32g+31 of its row in the block, as two
// 16-byte halves.  MFMA q of the block takes bytes 32g + 8q .. 32g + 8q + 7
// of every row of both operands (the order of K inside a block only has to
// be the same for both).
struct Block {
  sm_v4i alo[2], ahi[2];  // A rows r16 and r16 + 16
  sm_v4i wlo[2], whi[2];  // W rows r16 and r16 + 16
  float sa[2];            // activation scales of those A rows
  float sw;               // weight scale of the tile's 128-column block
};

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void gemm_small_kernel(const uint8_t* a, const float* a_scales, const uint8_t* w,
                                                         const float* w_scales, int m, int n, int k, void* c,
                                                         int64_t ldc, bool vec_c, int tiles_n) {
  __shared__ float red[kWaves][16][64];  // [wave][fragment * 4 + element][lane]

  const int tm = (int)blockIdx.x / tiles_n;
  const int tn = (int)blockIdx.x - tm * tiles_n;
  const int m0 = tm * kTile, n0 = tn * kTile;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r16 = lane & 15, grp = lane >> 4;
  const int nkb = k >> 7;

  // Buffers cover exactly the tile's rows of each operand and scale array,
  // so rows past m or n read as zero (the hardware range check, which also
  // skips the access).  Byte offsets fit in 32 bits: every operand is below
  // 2 GiB.
  const int arows = min(kTile, m - m0), wrows = min(kTile, n - n0);
  const uint32_t rowb = (uint32_t)k;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a + (size_t)m0 * rowb), 0, (int)((uint32_t)arows * rowb), kRsrcFlagsSmall);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + (size_t)n0 * rowb), 0, (int)((uint32_t)wrows * rowb), kRsrcFlagsSmall);
  const __amdgpu_buffer_rsrc_t sa_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a_scales + (size_t)m0 * nkb), 0, (int)((uint32_t)arows * (uint32_t)nkb * 4u), kRsrcFlagsSmall);
  // the 32 columns lie in one 128-column weight block (n0 is a multiple of 32)
  const __amdgpu_buffer_rsrc_t sw_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w_scales + (size_t)(n0 >> 7) * nkb), 0, (int)((uint32_t)nkb * 4u), kRsrcFlagsSmall);

  const uint32_t off0 = (uint32_t)r16 * rowb + 32u * (uint32_t)grp;
  const uint32_t off1 = off0 + 16u * rowb;
  const uint32_t soff0 = (uint32_t)r16 * (uint32_t)nkb * 4u;
  const uint32_t soff1 = soff0 + 16u * (uint32_t)nkb * 4u;
  auto load = [&](int kb, Block& b) {
    const int kofs = kb * 128;
    b.alo[0] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, (int)off0, kofs, 0));
    b.ahi[0] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, (int)off0 + 16, kofs, 0));
    b.alo[1] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, (int)off1, kofs, 0));
    b.ahi[1] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, (int)off1 + 16, kofs, 0));
    b.wlo[0] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, (int)off0, kofs, 0));
    b.whi[0] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, (int)off0 + 16, kofs, 0));
    b.wlo[1] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, (int)off1, kofs, 0));
    b.whi[1] = __builtin_bit_cast(sm_v4i, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, (int)off1 + 16, kofs, 0));
    b.sa[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sa_rsrc, (int)soff0, kb * 4, 0));
    b.sa[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sa_rsrc, (int)soff1, kb * 4, 0));
    b.sw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sw_rsrc, 0, kb * 4, 0));
  };

  sm_v4f acc[2][2];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[f][j] = sm_v4f{0.f, 0.f, 0.f, 0.f};

  // The MFMA forms the transposed fragment (W rows as its first operand), so
  // lane l holds C[m0 + 16f + r16][n0 + 16j + 4g + v], v = 0..3.
  auto multiply = [&](const Block& b) {
    sm_v4f p[2][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sm_v8bf wb[2], ab[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const sm_v4i& wr = q < 2 ? b.wlo[i] : b.whi[i];
        const sm_v4i& ar = q < 2 ? b.alo[i] : b.ahi[i];
        wb[i] = small_e4m3x8_to_bf16(wr[(q & 1) * 2], wr[(q & 1) * 2 + 1]);
        ab[i] = small_e4m3x8_to_bf16(ar[(q & 1) * 2], ar[(q & 1) * 2 + 1]);
      }
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          p[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[j], ab[f], q == 0 ? sm_v4f{0.f, 0.f, 0.f, 0.f}
                                                                                 : p[f][j], 0, 0, 0);
    }
    // the promotion: the block's partial times its two scales, into FP32
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const float s = b.sa[f] * b.sw;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][j][v] = __builtin_fmaf(p[f][j][v], s, acc[f][j][v]);
    }
  };

  // K blocks wave, wave + 4, ...: the next one is in flight while the
  // current one is multiplied
  if (wave < nkb) {
    Block cur, nxt;
    load(wave, cur);
    int kb = wave;
    for (; kb + kWaves < nkb; kb += kWaves) {
      load(kb + kWaves, nxt);
      multiply(cur);
      cur = nxt;
    }
    multiply(cur);
  }

  // fixed-order sum of the four waves' accumulators
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][(f * 2 + j) * 4 + v][lane] = acc[f][j][v];
  __syncthreads();
  const int f = wave >> 1, j = wave & 1;  // the fragment this wave stores
  sm_v4f r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = (f * 2 + j) * 4 + v;
    r[v] = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
  }

  const int row = m0 + f * 16 + r16;
  const int col = n0 + j * 16 + 4 * grp;
  if (row >= m) return;
  if constexpr (BF16_OUT) {
    uint16_t* crow = reinterpret_cast<uint16_t*>(c) + (int64_t)row * ldc;
    if (col + 3 < n && vec_c) {
      uint2 pk;
      pk.x = bf16_rne_bits(r[0]) | (bf16_rne_bits(r[1]) << 16);
      pk.y = bf16_rne_bits(r[2]) | (bf16_rne_bits(r[3]) << 16);
      *reinterpret_cast<uint2*>(crow + col) = pk;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col + v < n) crow[col + v] = (uint16_t)bf16_rne_bits(r[v]);
    }
  } else {
    float* crow = reinterpret_cast<float*>(c) + (int64_t)row * ldc;
    if (col + 3 < n && vec_c) {
      *reinterpret_cast<sm_v4f*>(crow + col) = r;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col + v < n) crow[col + v] = r[v];
    }
  }
}

}  // namespace

hipError_t launch_gemm_small(const uint8_t* a, const float* a_scales, const uint8_t* w, const float* w_scales,
                             int m, int n, int k, bool bf16_out, void* c, int64_t ldc, hipStream_t stream) {
  const int tiles_n = (n + kTile - 1) / kTile;
  const int64_t tiles = (int64_t)((m + kTile - 1) / kTile) * tiles_n;  // the caller keeps this small
  const bool vec_c = (ldc % 4) == 0;
  if (bf16_out) {
    hipLaunchKernelGGL(gemm_small_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, stream, a, a_scales, w,
                       w_scales, m, n, k, c, ldc, vec_c, tiles_n);
  } else {
    hipLaunchKernelGGL(gemm_small_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, stream, a, a_scales, w,
                       w_scales, m, n, k, c, ldc, vec_c, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace fp8q
