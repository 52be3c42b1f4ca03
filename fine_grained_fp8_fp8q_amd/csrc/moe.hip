// The steps on either side of the grouped expert GEMMs on one device
// (HBM-bound streaming kernels for gfx950).
//
// * FP8 dispatch gather (jp-study.kr doc 258368 ¶1): the activation is
//   quantized once, before the MoE dispatch, so the rows that go to the
//   hosted experts are copied as E4M3 codes plus their 1x128 scales -- 1 byte
//   per element instead of the 2 of BF16 -- straight into the expert-sorted
//   layout the grouped GEMM reads.
// * SwiGLU + quantize (tmdrlife.com wr_id=13334 ¶3-¶4): the MoE's SwiGLU
//   sits between the up- and the down-projection.  One pass reads the
//   up-projection output (gate | up halves) once, forms silu(g) * u in
//   float32, rounds it to BF16 and writes its 1x128 E4M3 quantization for
//   the down-projection; on request it also writes the 1x128 quantization of
//   the input itself (the pages cache SwiGLU inputs in FP8 with power-of-two
//   scales and recompute the output in the backward pass).  Without the
//   fusion the same work reads the input, writes BF16, reads it back and
//   writes codes: 9 bytes per output element instead of 5.
#include "fp8q_internal.h"
#include "quant_common.h"

namespace fp8q {

// ---------------------------------------------------------------- gather ---
// One wave per output row: its codes in 16-byte chunks (four chunks in
// flight per lane), then its scales.  The source index is wave-uniform.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ codes, int rows,
                                                          int cols, int64_t ldc, const float* __restrict__ scales,
                                                          int nb, const int32_t* __restrict__ index, int n_out,
                                                          uint8_t* __restrict__ out, int64_t ldo,
                                                          float* __restrict__ out_scales, bool vec) {
  const int lane = threadIdx.x & 63;
  const int i = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (i >= n_out) return;
  const int src = index[i];
  const bool valid = src >= 0 && src < rows;
  const uint8_t* s = codes + (valid ? (int64_t)src * ldc : 0);
  uint8_t* d = out + (int64_t)i * ldo;
  if (vec) {
    const int chunks = cols >> 4;
    for (int c0 = lane; c0 < chunks; c0 += 256) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u;
        v[u] = (valid && c < chunks) ? *reinterpret_cast<const uint4*>(s + 16 * c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u;
        if (c < chunks) st_stream16(d + 16 * c, v[u]);
      }
    }
  } else {
    for (int c = lane; c < cols; c += 64) d[c] = valid ? s[c] : (uint8_t)0;
  }
  const float* ss = scales + (valid ? (int64_t)src * nb : 0);
  float* ds = out_scales + (int64_t)i * nb;
  for (int j = lane; j < nb; j += 64) ds[j] = valid ? ss[j] : 0.0f;
}

// -------------------------------------------------------- SwiGLU + quant ---
// silu(g) * u in float32.  sigma(g) is formed from t = exp(-|g|) in (0, 1],
// which neither overflows nor loses the tail for large negative g:
// sigma(g) = 1 / (1 + t) for g >= 0 and t / (1 + t) for g < 0.  1 + t lies
// in [1, 2], where the hardware reciprocal is within 1 ulp.
// e^x for x <= 0: x log2(e) = n + f with |f| <= 1/2, reduced with log2(e)
// carried as a float32 head and a small tail (Cody and Waite's two-constant
// argument reduction, taken in base 2), 2^f from the hardware exp2, scaled by
// 2^n with ldexp (which also rounds subnormal results); below -104 the
// result is 0.
__device__ __forceinline__ float exp_nonpos(float x) {
  x = __builtin_fmaxf(x, -104.0f);
  const float l2e_hi = 1.44269502162933349609375f;  // RN32(log2 e)
  const float l2e_lo = 1.92596298909109e-8f;        // log2 e - l2e_hi
  const float n = __builtin_rintf(x * l2e_hi);
  const float f = __builtin_fmaf(x, l2e_lo, __builtin_fmaf(x, l2e_hi, -n));
  return __builtin_ldexpf(__builtin_amdgcn_exp2f(f), (int)n);
}

__device__ __forceinline__ float swiglu(float g, float u) {
  const float t = exp_nonpos(-__builtin_fabsf(g));
  const float r = __builtin_amdgcn_rcpf(1.0f + t);
  const float sg = g >= 0.0f ? r : t * r;
  return (g * sg) * u;
}

// The same value for gates g >= -64 in fewer instructions.  log2(e) is split
// as c1 + (log2(e) - c1) with c1 = 47274 / 2^15, its rounding to 16
// significant bits, so g * c1 is exact for every BF16 g (8 significant
// bits): e^-g = 2^(-g c1) * e^(-g k), k = 1 - c1 ln 2 = 4.888e-6, is one
// hardware exp2 of an exact argument times a factor within 3.2e-4 of 1,
// taken to first order by one fused multiply-add (the dropped second-order
// term is below 0.83 * 2^-24 relative for |g| <= 64).  sigma(g) =
// 1 / (1 + e^-g) needs no case split: for g in [-64, 0) e^-g stays below
// 2^93, and for large positive g it vanishes and 1 + e^-g is 1.
__device__ __forceinline__ float swiglu_direct(float g, float u) {
  constexpr float c1 = 47274.0f / 32768.0f;
  constexpr float k = 4.8884954e-06f;  // RN32(1 - c1 ln 2)
  const float e1 = __builtin_amdgcn_exp2f(g * -c1);
  const float e = __builtin_fmaf(-(g * k), e1, e1);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return (g * r) * u;
}

// Whether any of eight BF16 gates lies below -64: as unsigned 16-bit
// patterns those are the ones above 0xC280 (the pattern of -64; NaN
// patterns count too, and take the general path).
__device__ __forceinline__ bool gate_below_m64(uint4 g) {
  const uint32_t m = pk_max_u16(pk_max_u16(g.x, g.y), pk_max_u16(g.z, g.w));
  return max(m & 0xFFFFu, m >> 16) > 0xC280u;
}

// Eight (gate, up) BF16 pairs -> eight BF16 SwiGLU values in chunk layout,
// each rounded to nearest even by the hardware convert (v_cvt_pk_bf16_f32,
// two values per instruction).  DIRECT: every gate is at least -64.
typedef __bf16 sw_v2bf __attribute__((ext_vector_type(2)));
template <bool DIRECT>
__device__ __forceinline__ uint4 swiglu8(uint4 g, uint4 u) {
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
  const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo, hi;
    if constexpr (DIRECT) {
      lo = swiglu_direct(bf16_lo(gw[i]), bf16_lo(uw[i]));
      hi = swiglu_direct(bf16_hi(gw[i]), bf16_hi(uw[i]));
    } else {
      lo = swiglu(bf16_lo(gw[i]), bf16_lo(uw[i]));
      hi = swiglu(bf16_hi(gw[i]), bf16_hi(uw[i]));
    }
    y[i] = __builtin_bit_cast(uint32_t, sw_v2bf{(__bf16)lo, (__bf16)hi});
  }
  return make_uint4(y[0], y[1], y[2], y[3]);
}

// Quantize one chunk of a tile (the tile spread over a 16-lane DPP row) and
// store its codes and, from the row's first lane, the tile scale.
template <bool POW2>
__device__ __forceinline__ void quant_store(uint4 v, bool full, bool valid, int nvalid, uint8_t* dst,
                                            float* sdst, int sub) {
  const uint32_t amax = dpp_max16(absmax8(v));
  const TileScale ts = tile_scale<POW2>(amax);
  const uint2 c = encode8<POW2>(v, ts);
  if (full) {
    st_stream8(dst, c);
  } else if (valid) {
    store8_masked(dst, c, nvalid);
  }
  if (sub == 0 && valid) *sdst = ts.s;
}

// A 16-lane DPP row owns one output tile (128 columns of inter): lane sub
// reads 8 gate and 8 up values.  Each wave covers 4 tiles per iteration
// (lane l: tile base + l/16) of a grid-stride loop and loads the next
// iteration's gate and up chunks before it works on the current ones: the
// kernel is bound by its float32 arithmetic as much as by HBM, and the next
// loads stay in flight through that arithmetic.
template <bool POW2, bool CACHE, bool CPOW2>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const uint16_t* __restrict__ x, int inter, int64_t ldx,
                                                           uint8_t* __restrict__ codes, int64_t ldc,
                                                           float* __restrict__ scales, uint8_t* __restrict__ ccodes,
                                                           int64_t ldcc, float* __restrict__ cscales, int nb,
                                                           int ntiles, bool vec) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int sub = lane & 15;
  // 32-bit unsigned tile indices: ntiles < 2^31 and the stride is at most
  // 4 * 4 * kMaxStreamGrid, so base + stride never wraps.
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t step = gridDim.x * 16u;

  struct Chunk {
    uint4 g, u;
    int row, col, nvalid;
    bool valid, full;
  };
  auto fetch = [&](uint32_t base, Chunk& c) {
    const uint32_t t = base + (uint32_t)grp;
    c.valid = t < (uint32_t)ntiles;
    c.row = c.valid ? (int)(t / (uint32_t)nb) : 0;
    const int cb = c.valid ? (int)(t - (uint32_t)c.row * (uint32_t)nb) : 0;
    c.col = cb * 128 + sub * 8;
    c.nvalid = c.valid ? inter - c.col : 0;
    c.full = vec && c.valid && (cb * 128 + 128 <= inter);
    const uint16_t* src = x + (int64_t)c.row * ldx + c.col;
    if (c.full) {
      c.g = ld_stream16(src);
      c.u = ld_stream16(src + inter);
    } else {
      c.g = load8_masked(src, c.nvalid);
      c.u = load8_masked(src + inter, c.nvalid);
    }
  };

  uint32_t base = wave * 4u;
  if (base >= (uint32_t)ntiles) return;  // (wave-uniform)
  Chunk cur;
  fetch(base, cur);
  for (; base < (uint32_t)ntiles; base += step) {
    Chunk nxt = cur;
    const uint32_t nbase = base + step;
    if (nbase < (uint32_t)ntiles) fetch(nbase, nxt);  // (wave-uniform)
    const int cb = cur.col >> 7;
    // the general form only where a gate of this wave's chunks is below -64
    // (wave-uniform branch)
    const uint4 y = __builtin_amdgcn_ballot_w64(gate_below_m64(cur.g)) == 0 ? swiglu8<true>(cur.g, cur.u)
                                                                          : swiglu8<false>(cur.g, cur.u);
    quant_store<POW2>(y, cur.full, cur.valid, cur.nvalid, codes + (int64_t)cur.row * ldc + cur.col,
                      scales + (int64_t)cur.row * nb + cb, sub);
    if constexpr (CACHE) {
      // inter is a multiple of 128 here: the gate chunk is input tile cb,
      // the up chunk input tile nb + cb of the same row
      uint8_t* cdst = ccodes + (int64_t)cur.row * ldcc + cur.col;
      float* sdst = cscales + (int64_t)cur.row * (2 * nb) + cb;
      quant_store<CPOW2>(cur.g, cur.full, cur.valid, cur.nvalid, cdst, sdst, sub);
      quant_store<CPOW2>(cur.u, cur.full, cur.valid, cur.nvalid, cdst + inter, sdst + nb, sub);
    }
    cur = nxt;
  }
}

namespace {

template <bool POW2, bool CACHE, bool CPOW2>
hipError_t launch_swiglu(const uint16_t* x, int rows, int inter, int64_t ldx, uint8_t* codes, int64_t ldc,
                         float* scales, uint8_t* ccodes, int64_t ldcc, float* cscales, hipStream_t stream) {
  const int nb = (inter + 127) / 128;
  const int ntiles = rows * nb;  // < 2^31 (checked by the entry point)
  const bool vec = (ldx % 8 == 0) && (inter % 8 == 0) && (ldc % 8 == 0) && (!CACHE || ldcc % 8 == 0);
  const int64_t waves = ((int64_t)ntiles + 3) / 4;
  hipLaunchKernelGGL((swiglu_quant_kernel<POW2, CACHE, CPOW2>), dim3(stream_grid(waves)), dim3(256), 0, stream, x,
                     inter, ldx, codes, ldc, scales, ccodes, ldcc, cscales, nb, ntiles, vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_rows(const uint8_t* codes, int rows, int cols, int64_t ldc, const float* scales,
                              const int32_t* index, int n_out, uint8_t* out, int64_t ldo, float* out_scales,
                              hipStream_t stream) {
  const int nb = (cols + 127) / 128;
  const bool vec = (cols % 16 == 0) && (ldc % 16 == 0) && (ldo % 16 == 0);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((n_out + 3) / 4), dim3(256), 0, stream, codes, rows, cols, ldc,
                     scales, nb, index, n_out, out, ldo, out_scales, vec);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t* x, int rows, int inter, int64_t ldx, bool pow2, uint8_t* codes,
                               int64_t ldc, float* scales, bool cache_pow2, uint8_t* ccodes, int64_t ldcc,
                               float* cscales, hipStream_t stream) {
  if (!ccodes) {
    return pow2 ? launch_swiglu<true, false, false>(x, rows, inter, ldx, codes, ldc, scales, nullptr, 0, nullptr, stream)
                : launch_swiglu<false, false, false>(x, rows, inter, ldx, codes, ldc, scales, nullptr, 0, nullptr, stream);
  }
  if (pow2) {
    return cache_pow2 ? launch_swiglu<true, true, true>(x, rows, inter, ldx, codes, ldc, scales, ccodes, ldcc, cscales, stream)
                      : launch_swiglu<true, true, false>(x, rows, inter, ldx, codes, ldc, scales, ccodes, ldcc, cscales, stream);
  }
  return cache_pow2 ? launch_swiglu<false, true, true>(x, rows, inter, ldx, codes, ldc, scales, ccodes, ldcc, cscales, stream)
                    : launch_swiglu<false, true, false>(x, rows, inter, ldx, codes, ldc, scales, ccodes, ldcc, cscales, stream);
}

}  // namespace fp8q
