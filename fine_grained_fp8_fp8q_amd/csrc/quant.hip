// Online max-abs E4M3 quantizers for gfx950 (HBM-bound streaming kernels).
//
// jp-study.kr doc 258368 ¶1: the max-abs is taken online per 1x128
// activation tile and per 128x128 weight block.  tmdrlife.com wr_id=13334 ¶1
// describes exactly this pass as a read of the BF16 values from HBM and a
// write of the FP8 values back; the kernels below make that round trip at
// close to HBM speed: one 16-byte load per lane per 8 elements, a DPP
// max-abs over the 16 lanes that hold one tile, and packed code stores.
#include <type_traits>

#include "fp8q_internal.h"
#include "quant_common.h"

namespace fp8q {

// ----------------------------------------------------------- 1x128 rows ---
// A 16-lane DPP row owns one tile (16 lanes x 8 BF16).  Each wave handles
// 16 consecutive tiles per iteration: load u (0..3) of lane l reads tile
// base + 4u + l/16, so every load instruction covers 4 consecutive tiles
// (1 KiB when they share a row).  The scales of a DPP row's four tiles are
// worked out once, lane u of the row taking tile u, and broadcast back to
// the row (row_newbcast): one scale computation per lane and iteration
// instead of four (the free scale is a corrected quotient and a corrected
// reciprocal, about 10 instructions).

// Tile u's scale state, from lane u of each DPP row.
template <bool POW2, int U>
__device__ __forceinline__ TileScale row_tile_scale(const TileScale& tm) {
  TileScale ts;
  ts.s = 0.0f;  // (stored by lane u itself)
  if constexpr (POW2) {
    ts.div = 1.0f;
    ts.mul = 1.0f;
    ts.xscale = 1.0f;
    ts.slow = false;
    ts.neg_e = (int)row_bcast<U>((uint32_t)tm.neg_e);
  } else {
    ts.div = row_bcast<U>(tm.div);
    ts.mul = row_bcast<U>(tm.mul);
    ts.neg_e = 0;
    ts.slow = row_bcast<U>((uint32_t)tm.slow) != 0u;
    ts.xscale = ts.slow ? 0x1p64f : 1.0f;
  }
  return ts;
}

template <bool POW2>
__device__ __forceinline__ void quant_rows_body(int bid, int nblocks, const uint16_t* __restrict__ x, int cols,
                                                int64_t ldx, uint8_t* __restrict__ codes, int64_t ldc,
                                                float* __restrict__ scales, int nb, int ntiles, bool vec) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int sub = lane & 15;
  // Tile indices count in 32-bit unsigned: ntiles < 2^31 and the stride is
  // at most 16 tiles x 8 waves x kMaxRowsGrid = 2^27, so base + stride never
  // wraps.  (Workgroups of 64 or 512 threads: 16 tiles per wave.)
  const uint32_t wave = ((uint32_t)bid * blockDim.x + threadIdx.x) >> 6;
  const uint32_t step = (uint32_t)nblocks * (blockDim.x >> 2);

  for (uint32_t base = wave * 16u; base < (uint32_t)ntiles; base += step) {
    uint4 v[4];
    int row[4], cb[4];
    bool valid[4], full[4];
    // tile base + 4u + grp is (row[u], cb[u]): one division, then steps of
    // four tiles (rows of at least four tiles) or a division per tile
    {
      const uint32_t t = base + (uint32_t)grp;
      row[0] = (int)(t / (uint32_t)nb);
      cb[0] = (int)(t - (uint32_t)row[0] * (uint32_t)nb);
    }
#pragma unroll
    for (int u = 1; u < 4; ++u) {
      if (nb >= 4) {
        const bool wrap = cb[u - 1] + 4 >= nb;
        cb[u] = cb[u - 1] + 4 - (wrap ? nb : 0);
        row[u] = row[u - 1] + (wrap ? 1 : 0);
      } else {
        const uint32_t t = base + (uint32_t)(4 * u + grp);
        row[u] = (int)(t / (uint32_t)nb);
        cb[u] = (int)(t - (uint32_t)row[u] * (uint32_t)nb);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      valid[u] = base + (uint32_t)(u * 4 + grp) < (uint32_t)ntiles;
      full[u] = vec && valid[u] && (cb[u] * 128 + 128 <= cols);
      const uint16_t* src = x + (int64_t)row[u] * ldx + cb[u] * 128 + sub * 8;
      if (full[u]) {
        v[u] = ld_stream16(src);
      } else {
        v[u] = load8_masked(src, valid[u] ? cols - (cb[u] * 128 + sub * 8) : 0);
      }
    }
    uint32_t am[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) am[u] = dpp_max16(absmax8(v[u]));
    // lane u (< 4) of each DPP row takes the row's tile u; the scale matrix
    // is [rows, nb] contiguous, so tile t's scale is scales[t]
    const uint32_t mine = sub == 1 ? am[1] : sub == 2 ? am[2] : sub == 3 ? am[3] : am[0];
    const TileScale tm = tile_scale<POW2>(mine);
    {
      const uint32_t ts_tile = base + (uint32_t)(4 * sub + grp);
      if (sub < 4 && ts_tile < (uint32_t)ntiles) scales[ts_tile] = tm.s;
    }
    auto encode_store = [&](int u, const TileScale& ts, auto enc) {
      const uint2 c = enc(v[u], ts);
      uint8_t* dst = codes + (int64_t)row[u] * ldc + cb[u] * 128 + sub * 8;
      if (full[u]) {
        st_stream8(dst, c);
      } else if (valid[u]) {
        store8_masked(dst, c, cols - (cb[u] * 128 + sub * 8));
      }
    };
    auto all4 = [&](auto enc) {
      encode_store(0, row_tile_scale<POW2, 0>(tm), enc);
      encode_store(1, row_tile_scale<POW2, 1>(tm), enc);
      encode_store(2, row_tile_scale<POW2, 2>(tm), enc);
      encode_store(3, row_tile_scale<POW2, 3>(tm), enc);
    };
    if constexpr (POW2) {
      all4([](uint4 x, const TileScale& t) { return encode8<true>(x, t); });
    } else if (__builtin_amdgcn_ballot_w64(sub < 4 && tm.slow) == 0) {
      // (one wave-uniform decision for the wave's 16 tiles)
      all4([](uint4 x, const TileScale& t) { return encode8_markstein<false>(x, t); });
    } else {
      all4([](uint4 x, const TileScale& t) { return encode8_markstein<true>(x, t); });
    }
  }
}

template <bool POW2>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int cols,
                                                         int64_t ldx, uint8_t* __restrict__ codes,
                                                         int64_t ldc, float* __restrict__ scales,
                                                         int nb, int ntiles, bool vec) {
  quant_rows_body<POW2>((int)blockIdx.x, (int)gridDim.x, x, cols, ldx, codes, ldc, scales, nb, ntiles, vec);
}

// ------------------------------------------------------ 128x128 blocks ---
// One workgroup (8 waves) per block.  Thread t holds rows t/16 + 32p
// (p = 0..3) of the block, 8 BF16 each, so the block is read once and kept
// in registers across the max-abs reduction.  Eight waves of four rows each
// measured faster than four waves of eight rows (7168 x 18432: 68.0 ->
// 66.6 us; 4096 x 7168: 17.3 -> 17.1 us; 300 x 1000: 8.6 -> 7.4 us).
constexpr int kBlockThreads = 512;
template <bool POW2>
__device__ __forceinline__ void quant_blocks_body(int bid, const uint16_t* __restrict__ w, int n, int k,
                                                  int64_t ldw, uint8_t* __restrict__ codes, int64_t ldc,
                                                  float* __restrict__ scales, int bk, bool vec) {
  constexpr int kWaves = kBlockThreads / 64, kRows = 128 / (kBlockThreads / 16);  // rows per thread
  __shared__ uint32_t red[kWaves];
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  const int r0 = tid >> 4;
  const int bi = bid / bk;
  const int bj = bid - bi * bk;
  const int row0 = bi * 128, col0 = bj * 128 + sub * 8;
  const bool full = vec && (row0 + 128 <= n) && (bj * 128 + 128 <= k);

  uint4 v[kRows];
#pragma unroll
  for (int p = 0; p < kRows; ++p) {
    const int r = row0 + r0 + (kBlockThreads / 16) * p;
    const uint16_t* src = w + (int64_t)r * ldw + col0;
    if (full) {
      v[p] = ld_stream16(src);
    } else {
      v[p] = load8_masked(src, r < n ? k - col0 : 0);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < kRows; ++p) m = max(m, absmax8(v[p]));
  m = dpp_max16(m);
  m = max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
          max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) m = max(m, red[i]);

  const TileScale ts = tile_scale<POW2>(m);
#pragma unroll
  for (int p = 0; p < kRows; ++p) {
    const int r = row0 + r0 + (kBlockThreads / 16) * p;
    const uint2 c = encode8<POW2>(v[p], ts);
    uint8_t* dst = codes + (int64_t)r * ldc + col0;
    if (full) {
      st_stream8(dst, c);
    } else if (r < n) {
      store8_masked(dst, c, k - col0);
    }
  }
  if (tid == 0) scales[bid] = ts.s;
}

template <bool POW2>
__global__ __launch_bounds__(kBlockThreads) void quant_blocks_kernel(const uint16_t* __restrict__ w, int n,
                                                           int k, int64_t ldw,
                                                           uint8_t* __restrict__ codes, int64_t ldc,
                                                           float* __restrict__ scales, int bk,
                                                           bool vec) {
  quant_blocks_body<POW2>((int)blockIdx.x, w, n, k, ldw, codes, ldc, scales, bk, vec);
}

// ------------------------------- both operands of a linear layer at once ---
// The activation's 1x128 tiles (the first `ga` workgroups, as in
// quant_rows_kernel) and the weight's 128x128 blocks (one workgroup each, as
// in quant_blocks_kernel) in one launch of 8-wave workgroups: one grid ramp
// and drain instead of two, and the two streams overlap.
template <bool PA, bool PW>
__global__ __launch_bounds__(kBlockThreads) void quant_linear_kernel(const uint16_t* __restrict__ x, int cols,
                                                                     int64_t ldx,
                                                           uint8_t* __restrict__ a_codes, int64_t lda,
                                                           float* __restrict__ a_scales, int nb, int ntiles,
                                                           bool avec, int ga, const uint16_t* __restrict__ w,
                                                           int n, int64_t ldw, uint8_t* __restrict__ w_codes,
                                                           int64_t ldwc, float* __restrict__ w_scales, int bk,
                                                           bool wvec) {
  if ((int)blockIdx.x < ga) {
    quant_rows_body<PA>((int)blockIdx.x, ga, x, cols, ldx, a_codes, lda, a_scales, nb, ntiles, avec);
  } else {
    quant_blocks_body<PW>((int)blockIdx.x - ga, w, n, cols, ldw, w_codes, ldwc, w_scales, bk, wvec);
  }
}

// ---------------------------------- 128x128 blocks, plus the transpose ---
// The same block quantization, also written transposed for the activation
// gradient dX = dY . W (jp-study.kr doc 258368 ¶3: all three GEMMs of a
// linear layer run in FP8), whose reduction axis is N: a square block's max-
// abs does not depend on orientation, so W^T quantized per block is exactly
// the transpose of W quantized.  Thread t owns the 8x8 sub-block at rows
// 8(t/16).., columns 8(t%16).., transposes its 64 codes in registers into
// an LDS copy of the transposed block, which then leaves as whole 128-byte
// W^T row segments.  `codes` may be null (only the transposed copy is
// written).
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

template <bool POW2>
__global__ __launch_bounds__(256) void quant_blocks_t_kernel(const uint16_t* __restrict__ w, int n,
                                                             int k, int64_t ldw,
                                                             uint8_t* __restrict__ codes, int64_t ldc,
                                                             float* __restrict__ scales,
                                                             uint8_t* __restrict__ codes_t, int64_t ldt,
                                                             float* __restrict__ scales_t, int bn, int bk,
                                                             bool vec) {
  constexpr int kTRowBytes = 144;  // 16-byte aligned rows of the transposed block
  __shared__ uint32_t red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile_t[128 * kTRowBytes];
  const int tid = threadIdx.x;
  const int sb = tid & 15;   // column group: columns 8sb..8sb+7 of the block
  const int sa = tid >> 4;   // row group: rows 8sa..8sa+7
  const int bi = blockIdx.x / bk;
  const int bj = blockIdx.x - bi * bk;
  const int row0 = bi * 128 + 8 * sa, col0 = bj * 128 + 8 * sb;
  const bool full = vec && (bi * 128 + 128 <= n) && (bj * 128 + 128 <= k);

  uint4 v[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = row0 + p;
    const uint16_t* src = w + (int64_t)r * ldw + col0;
    if (full) {
      v[p] = ld_stream16(src);
    } else {
      v[p] = load8_masked(src, r < n ? k - col0 : 0);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) m = max(m, absmax8(v[p]));
  m = dpp_max16(m);
  m = max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
          max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));

  const TileScale ts = tile_scale<POW2>(m);
  uint2 c[8];  // codes of rows row0 + p, columns col0..col0+7
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    c[p] = encode8<POW2>(v[p], ts);
    if (codes) {
      const int r = row0 + p;
      uint8_t* dst = codes + (int64_t)r * ldc + col0;
      if (full) {
        st_stream8(dst, c[p]);
      } else if (r < n) {
        store8_masked(dst, c[p], k - col0);
      }
    }
  }
  // column j of the sub-block (byte j of every row's codes) goes to LDS as
  // row 8sb + j of the transposed block; the block then leaves as whole
  // 128-byte W^T row segments (8 lanes per segment, 16 bytes each).  The
  // 16-byte chunks of a row are rotated by sb/2, so the 32 lanes of a
  // half-wave write 64 distinct banks (unrotated, every second sb lands on
  // the same two bank offsets).
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      lo |= byte_of(j < 4 ? c[p].x : c[p].y, j & 3) << (8 * p);
      hi |= byte_of(j < 4 ? c[p + 4].x : c[p + 4].y, j & 3) << (8 * p);
    }
    *reinterpret_cast<uint2*>(&tile_t[(8 * sb + j) * kTRowBytes + 8 * ((sa + 2 * (sb >> 1)) & 15)]) =
        make_uint2(lo, hi);
  }
  __syncthreads();
  const int brow0 = bi * 128, bcol0 = bj * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int tr = q >> 3, ch = q & 7;   // transposed row (a column of W), 16-byte chunk
    const uint4 val = *reinterpret_cast<const uint4*>(&tile_t[tr * kTRowBytes + 16 * ((ch + (tr >> 4)) & 7)]);
    const int col = bcol0 + tr;
    uint8_t* dst = codes_t + (int64_t)col * ldt + brow0 + 16 * ch;
    if (full) {
      st_stream16(dst, val);
    } else if (col < k) {
      store8_masked(dst, make_uint2(val.x, val.y), n - (brow0 + 16 * ch));
      store8_masked(dst + 8, make_uint2(val.z, val.w), n - (brow0 + 16 * ch + 8));
    }
  }
  if (tid == 0) {
    if (scales) scales[blockIdx.x] = ts.s;
    scales_t[bj * bn + bi] = ts.s;
  }
}

// Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i % 8).
// This maps them so that each XCD runs one contiguous range of logical
// blocks: the token blocks of a feature group follow one another on one XCD,
// and the 4-byte scales they write, adjacent in each feature's scale row,
// meet in that XCD's L2 as whole lines instead of reaching memory as
// partial-line writes from eight L2s.
__device__ __forceinline__ int xcd_block(int bid, int nblk) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return xcd * per + min(xcd, rem) + idx;
}

// --------------------------------------------- 128x1 token-axis tiles ---
// Workgroup tile: 128 tokens (rows of x) x 64 features (columns of x); the
// token block varies fastest along the logical block index.
// Thread (q = tid/8, c8 = tid%8) loads tokens 4q..4q+3, features 8c8..8c8+7,
// so for each feature it holds four consecutive tokens: one code word.  The
// per-feature max-abs runs over the 32 threads sharing c8; codes go through
// LDS ([feature][token], 144-byte rows) and leave feature-major, 128 tokens
// (one 128-byte line) per feature.  Within a row the token words are rotated
// by 8 words per group of 8 features: the 64 lanes that write one word each
// (8 feature groups x 8 token words) then hit 64 distinct banks, where the
// unrotated rows put every feature group on the same two bank offsets.
// rot4: the feature group turns with the token block inside aligned groups of
// four feature groups.  With rows 4 KB apart (2048 features) the ~256
// workgroups resident on an XCD otherwise read only about two distinct
// 128-byte column offsets of every row; spreading them over four measured
// 22.5 -> 21.3 us at 16384 x 2048 on MI355X.  The launcher sets it only when
// every XCD's range of blocks holds whole groups, so each feature's scale
// line is still written from one L2.
template <bool POW2>
__global__ __launch_bounds__(256) void quant_token_t_kernel(const uint16_t* __restrict__ x, int rows,
                                                            int cols, int64_t ldx,
                                                            uint8_t* __restrict__ codes, int64_t ldc,
                                                            float* __restrict__ scales, int ntb,
                                                            bool vec, bool rot4) {
  constexpr int kRowBytes = 144;  // 16-byte aligned rows for the store reads
  __shared__ uint32_t red[4][64];
  // per-feature scale state, read back 8 features (32 bytes) at a time
  __shared__ __attribute__((aligned(16))) float s_div[64];
  __shared__ __attribute__((aligned(16))) float s_mul[64];
  __shared__ __attribute__((aligned(16))) int s_nege[64];
  __shared__ unsigned char s_slow[64];
  __shared__ int s_anyslow;  // some feature of the block has a tiny amax
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * kRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c8 = tid & 7;
  const int q = tid >> 3;  // 0..31
  const int logical = xcd_block(blockIdx.x, gridDim.x);
  const int tb = logical % ntb;
  const int t0 = tb * 128;
  int fg = logical / ntb;
  if (rot4) fg = (fg & ~3) | ((fg + tb) & 3);
  const int f0 = fg * 64;
  const bool full = vec && (t0 + 128 <= rows) && (f0 + 64 <= cols);

  uint4 v[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int t = t0 + 4 * q + p;
    const uint16_t* src = x + (int64_t)t * ldx + f0 + 8 * c8;
    if (full) {
      v[p] = ld_stream16(src);
    } else {
      v[p] = load8_masked(src, t < rows ? cols - (f0 + 8 * c8) : 0);
    }
  }
  // per-feature max-abs over this thread's 4 tokens, packed two features per word
  const uint32_t k = 0x7FFF7FFFu;
  uint32_t m[4];
  m[0] = pk_max_u16(pk_max_u16(v[0].x & k, v[1].x & k), pk_max_u16(v[2].x & k, v[3].x & k));
  m[1] = pk_max_u16(pk_max_u16(v[0].y & k, v[1].y & k), pk_max_u16(v[2].y & k, v[3].y & k));
  m[2] = pk_max_u16(pk_max_u16(v[0].z & k, v[1].z & k), pk_max_u16(v[2].z & k, v[3].z & k));
  m[3] = pk_max_u16(pk_max_u16(v[0].w & k, v[1].w & k), pk_max_u16(v[2].w & k, v[3].w & k));
  // across the 8 lanes of the wave with the same c8 (lane bits 3..5):
  // lane l ^ 8 is lane l rotated by 8 within its 16-lane DPP row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = pk_max_u16(m[i], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m[i], 0x128, 0xF, 0xF, false));
    m[i] = pk_max_u16(m[i], (uint32_t)__shfl_xor((int)m[i], 16));
    m[i] = pk_max_u16(m[i], (uint32_t)__shfl_xor((int)m[i], 32));
  }
  if (tid == 0) s_anyslow = 0;
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wave][8 * c8 + 2 * i] = m[i] & 0xFFFFu;
      red[wave][8 * c8 + 2 * i + 1] = m[i] >> 16;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const uint32_t a = max(max(red[0][tid], red[1][tid]), max(red[2][tid], red[3][tid]));
    const TileScale ts = tile_scale<POW2>(a);
    s_div[tid] = ts.div;
    s_mul[tid] = ts.mul;
    s_nege[tid] = ts.neg_e;
    s_slow[tid] = ts.slow;
    if (ts.slow) s_anyslow = 1;
    if (f0 + tid < cols) scales[(int64_t)(f0 + tid) * ntb + tb] = ts.s;
  }
  __syncthreads();

  // encode: feature 8*c8 + j, tokens 4q..4q+3 -> one word at tile[f][4q].
  // The thread's 8 features' scale state comes in as whole 16-byte LDS
  // reads; the scaling of x by 2^64 for a tiny-amax feature is taken only
  // when the block has one (a workgroup-uniform branch), so the common case
  // is the bare Markstein quotient.
  auto word_of = [&](int p, int j) {
    return (j >> 1) == 0 ? v[p].x : (j >> 1) == 1 ? v[p].y : (j >> 1) == 2 ? v[p].z : v[p].w;
  };
  auto put = [&](int j, uint32_t w) {
    const int f = 8 * c8 + j;
    *reinterpret_cast<uint32_t*>(&tile[f * kRowBytes + 4 * ((q + 8 * c8) & 31)]) = w;
  };
  if constexpr (POW2) {
    const int4 n0 = *reinterpret_cast<const int4*>(&s_nege[8 * c8]);
    const int4 n1 = *reinterpret_cast<const int4*>(&s_nege[8 * c8 + 4]);
    const int ne[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float e[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t word = word_of(p, j);
        e[p] = __builtin_ldexpf((j & 1) ? bf16_hi(word) : bf16_lo(word), ne[j]);
      }
      put(j, pack4_e4m3(e[0], e[1], e[2], e[3]));
    }
  } else {
    const float4 d0 = *reinterpret_cast<const float4*>(&s_div[8 * c8]);
    const float4 d1 = *reinterpret_cast<const float4*>(&s_div[8 * c8 + 4]);
    const float4 r0 = *reinterpret_cast<const float4*>(&s_mul[8 * c8]);
    const float4 r1 = *reinterpret_cast<const float4*>(&s_mul[8 * c8 + 4]);
    const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    const float ml[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    if (s_anyslow == 0) {  // (workgroup-uniform)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t word = word_of(p, j);
          const float xv = (j & 1) ? bf16_hi(word) : bf16_lo(word);
          const float q0 = xv * ml[j];
          const float er = __builtin_fmaf(-q0, dv[j], xv);
          e[p] = __builtin_copysignf(__builtin_fmaf(er, ml[j], q0), xv);
        }
        put(j, pack4_e4m3(e[0], e[1], e[2], e[3]));
      }
    } else {
      // a tiny-amax feature scales its x by 2^64 (its divisor already is)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        TileScale ts;
        ts.div = dv[j];
        ts.mul = ml[j];
        ts.neg_e = 0;
        ts.slow = s_slow[8 * c8 + j] != 0;
        ts.xscale = ts.slow ? 0x1p64f : 1.0f;
        float e[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t word = word_of(p, j);
          e[p] = quotient_free((j & 1) ? bf16_hi(word) : bf16_lo(word), ts);
        }
        put(j, pack4_e4m3(e[0], e[1], e[2], e[3]));
        // (one feature at a time: this rare path keeps the fast path's
        // register budget)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();

  // store: 8 consecutive lanes write one feature row's 128 token bytes, so
  // each store instruction covers 8 whole 128-byte row segments (spreading a
  // row over lanes of different instructions measured 25% slower)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int f = (tid >> 3) + 32 * it;
    const int ch = tid & 7;
    const uint4 w = *reinterpret_cast<const uint4*>(&tile[f * kRowBytes + 16 * ((ch + 2 * (f >> 3)) & 7)]);
    uint8_t* dst = codes + (int64_t)(f0 + f) * ldc + t0 + 16 * ch;
    if (full) {
      st_stream16(dst, w);
    } else if (f0 + f < cols) {
      const int nvalid = rows - (t0 + 16 * ch);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < nvalid) dst[i] = (uint8_t)((ww[i >> 2] >> (8 * (i & 3))) & 0xFF);
      }
    }
  }
}

// ------------------------------------------------------------ launchers ---
// rows_grid (fp8q_internal.h): one pass per wave (16 tiles per wave) up to
// 2^20 workgroups; a large grid keeps more loads in flight than a
// grid-stride loop over a capped grid (measured on MI355X: 4.7 TB/s at 2048
// workgroups vs 5.8 TB/s with one pass for this 2:1 read:write stream).  The
// row quantizer launches one-wave workgroups: 16.5 -> 16.0 us at 4096 x 7168
// and 6.0 -> 5.75 us at 3773 x 2048 against four-wave ones (no change at
// 16384 x 7168); the combined linear launch uses the 8-wave workgroups its
// weight blocks take.

hipError_t launch_quant_rows(const uint16_t* x, int rows, int cols, int64_t ldx, bool pow2,
                             uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream) {
  const int nb = (cols + 127) / 128;
  const int ntiles = rows * nb;
  const dim3 grid(rows_grid(ntiles, 16)), block(64);
  const bool vec = ldx % 8 == 0 && ldc % 8 == 0;  // 16-byte loads, 8-byte stores
  if (pow2) {
    hipLaunchKernelGGL(quant_rows_kernel<true>, grid, block, 0, stream, x, cols, ldx, codes, ldc, scales, nb, ntiles, vec);
  } else {
    hipLaunchKernelGGL(quant_rows_kernel<false>, grid, block, 0, stream, x, cols, ldx, codes, ldc, scales, nb, ntiles, vec);
  }
  return hipGetLastError();
}

hipError_t launch_quant_blocks(const uint16_t* w, int n, int k, int64_t ldw, bool pow2,
                               uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream) {
  const int bn = (n + 127) / 128, bk = (k + 127) / 128;
  const dim3 grid(bn * bk), block(kBlockThreads);
  const bool vec = ldw % 8 == 0 && ldc % 8 == 0;
  if (pow2) {
    hipLaunchKernelGGL(quant_blocks_kernel<true>, grid, block, 0, stream, w, n, k, ldw, codes, ldc, scales, bk, vec);
  } else {
    hipLaunchKernelGGL(quant_blocks_kernel<false>, grid, block, 0, stream, w, n, k, ldw, codes, ldc, scales, bk, vec);
  }
  return hipGetLastError();
}

hipError_t launch_quant_linear(const uint16_t* x, int m, int k, int64_t ldx, bool a_pow2, uint8_t* a_codes,
                               int64_t lda, float* a_scales, const uint16_t* w, int n, int64_t ldw, bool w_pow2,
                               uint8_t* w_codes, int64_t ldwc, float* w_scales, hipStream_t stream) {
  const int nb = (k + 127) / 128;
  const int ntiles = m * nb;
  const int ga = m > 0 ? rows_grid(ntiles, kBlockThreads / 4) : 0;
  const int bn = (n + 127) / 128;
  const int gw = n > 0 ? bn * nb : 0;
  const bool avec = ldx % 8 == 0 && lda % 8 == 0;
  const bool wvec = ldw % 8 == 0 && ldwc % 8 == 0;
  const dim3 grid(ga + gw), block(kBlockThreads);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, stream, x, k, ldx, a_codes, lda, a_scales, nb, ntiles, avec, ga, w,
                       n, ldw, w_codes, ldwc, w_scales, nb, wvec);
  };
  if (a_pow2) {
    if (w_pow2) go(quant_linear_kernel<true, true>); else go(quant_linear_kernel<true, false>);
  } else {
    if (w_pow2) go(quant_linear_kernel<false, true>); else go(quant_linear_kernel<false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_quant_blocks_t(const uint16_t* w, int n, int k, int64_t ldw, bool pow2,
                                 uint8_t* codes, int64_t ldc, float* scales, uint8_t* codes_t,
                                 int64_t ldt, float* scales_t, hipStream_t stream) {
  const int bn = (n + 127) / 128, bk = (k + 127) / 128;
  const dim3 grid(bn * bk), block(256);
  const bool vec = ldw % 8 == 0 && (codes == nullptr || ldc % 8 == 0) && ldt % 16 == 0;
  if (pow2) {
    hipLaunchKernelGGL(quant_blocks_t_kernel<true>, grid, block, 0, stream, w, n, k, ldw, codes, ldc, scales,
                       codes_t, ldt, scales_t, bn, bk, vec);
  } else {
    hipLaunchKernelGGL(quant_blocks_t_kernel<false>, grid, block, 0, stream, w, n, k, ldw, codes, ldc, scales,
                       codes_t, ldt, scales_t, bn, bk, vec);
  }
  return hipGetLastError();
}

hipError_t launch_quant_token_t(const uint16_t* x, int rows, int cols, int64_t ldx, bool pow2,
                                uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream) {
  const int ntb = (rows + 127) / 128;
  const int nblk = ntb * ((cols + 63) / 64);
  const dim3 grid(nblk), block(256);
  const bool vec = ldx % 8 == 0 && ldc % 16 == 0;  // 16-byte loads and stores
  // every XCD's contiguous range of blocks (xcd_block) is whole groups of
  // four feature groups: rotation stays inside one XCD
  const bool rot4 = nblk % 8 == 0 && (nblk / 8) % (4 * ntb) == 0;
  if (pow2) {
    hipLaunchKernelGGL(quant_token_t_kernel<true>, grid, block, 0, stream, x, rows, cols, ldx, codes, ldc, scales, ntb, vec,
                       rot4);
  } else {
    hipLaunchKernelGGL(quant_token_t_kernel<false>, grid, block, 0, stream, x, rows, cols, ldx, codes, ldc, scales, ntb, vec,
                       rot4);
  }
  return hipGetLastError();
}

}  // namespace fp8q
