// Block-scaled FP8 (E4M3) GEMMs for gfx950: dense, grouped (MoE experts) and
// weight gradient.
//
// What is computed (tmdrlife.com wr_id=13334 ¶3; gnrental.net wr_id=40936
// ¶4; jp-study.kr doc 258368 ¶3): partial sums over 128 elements of K of
// E4M3 x E4M3 products, each multiplied by its activation and weight scales
// and added into FP32 accumulators.
//
// Accumulation precision.  tmdrlife.com wr_id=13334 ¶2 warns that the FP8
// matrix units of the pages' hardware accumulate in limited-width fixed
// point.  The FP8 MFMAs of gfx950 (16x16x128 and 32x32x64 f8f6f4, and the
// 16x16x32 fp8 form) behave the same way: measured over one 128-element
// block of random E4M3 codes whose exponents spread over +-4 binades, their
// error reaches 5e-5 of sum|a*b| (1e-4 at +-7), far above float32
// accumulation (< 4e-7).  The BF16 MFMA accumulates at float32 grade, and
// every E4M3 value is exactly a BF16 value.  So the operands stay E4M3 in
// HBM and LDS (half the bytes of BF16) and each fragment is widened to BF16
// in registers (v_cvt_scalef32_pk_bf16_fp8 with scale 1, exact) right before
// v_mfma_f32_16x16x32_bf16.  Four chained MFMAs cover one 128-element block;
// their float32 result is the block's partial, folded with one v_fma_f32 per
// element (the pages' "promotion"), while the MFMAs of the next fragment run.
//
// Workgroup tile 256 x 256 x 128, 8 waves (4 along M x 2 along N: two per
// SIMD, so one wave's LDS waits and conversions overlap the other's MFMAs),
// wave tile 64 x 128 in at most 256 registers.  The MFMA computes the
// transposed tile (W rows as its A operand, A rows as its B operand), so
// each lane owns one output row m and four consecutive columns n: with 1x128
// activation scales and 128x128 weight blocks the fold scale a[m] * w[n/128]
// is one value per lane and per 16-row M fragment.
//
// Data movement: both operands are K-contiguous (A [M,K], W [N,K]).  Each
// 128-byte K slice of a row is moved global->LDS by buffer_load_dwordx4 with
// an LDS destination (no VGPR staging), 8 rows per wave instruction, with
// the 16-byte chunks of a row XOR-swizzled so the fragment reads
// (ds_read_b128, 16 rows at the same chunk) hit distinct banks.  Lane group
// g (lanes 16g..16g+15) reads bytes 32g..32g+31 of its row; the k order
// inside a block only has to be the same for both operands.  Two LDS stages
// (65 KiB each): K block kb+1 streams in while kb is multiplied; one barrier
// per K block.  Grouped tiles of at most 128 rows use three smaller stages
// (two K blocks in flight).  The row and column scales go through their own
// double buffer, four K blocks at a time, a quarter of the next group with
// every K block's refill.
//
// Output: float32, BF16 (nearest even), or -- dense only -- the BF16 value
// quantized per 1x128 tile along N (E4M3 codes + float32 scales), the form a
// following FP8 GEMM reads (tmdrlife.com wr_id=13334 ¶1).
#include <atomic>
#include <type_traits>

#include "fp8q_internal.h"
#include "quant_common.h"

namespace fp8q {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 512;
// A stage holds one K block: the A rows of the tile (128 B each) and the
// 256 W rows; a full tile's stage also holds the weight gradient's W scales
// of the block, one per column [256].  A full tile's stage is 65 KiB (two
// stages); a grouped tile of at most 128 (64) rows has a 16 (8) KiB A part,
// so three of its stages fit in 144 KiB.
template <int AROWS>
struct StageLayout {
  static constexpr int kW = AROWS * BK;            // W rows start here
  static constexpr int kS = kW + BN * BK;          // weight-gradient W scales (full tiles)
  static constexpr int kBytes = kS + (AROWS == BM ? BN * 4 : 0);
};
constexpr int kFullStage = StageLayout<BM>::kBytes;     // 65 KiB
constexpr int kSmallStage = StageLayout<128>::kBytes;   // 48 KiB (also holds the 64-row layout)
// The other scales live in their own double buffer after the stages: half
// h holds one group of four K blocks, [256 A rows | 256 W columns] x 4
// blocks (one W value per column: the scale of its 128-column block).  A
// load that brings one block of 256 row scales touches 256 cache lines (the
// scale rows are K/128 floats apart), against 512 for the block's operand
// rows; a load of four blocks of 16 rows touches 16.
constexpr int kSclHalf = (BM + BN) * 4 * 4;             // 8 KiB
constexpr int kSclBytes = 2 * kSclHalf;

enum Mode { kDense = 0, kGrouped = 1, kWgrad = 2 };
// Output forms: float32, BF16 (RNE), or the BF16 value quantized per 1x128
// tile along N to E4M3 codes plus float32 scales (free or power-of-two).
enum Out { kOutF32 = 0, kOutBF16 = 1, kOutE4M3 = 2, kOutE4M3Pow2 = 3 };

// Buffer resource word 3 for raw (untyped, unswizzled) buffer access.
constexpr int kRsrcFlags = 0x00020000;

struct GemmArgs {
  const uint8_t* a;       // codes [rows, k]
  const float* sa;        // [rows, k/128]
  const uint8_t* w;       // codes [(groups,) n, k]
  const float* sw;        // dense/grouped: [(groups,) ceil(n/128), k/128]; wgrad: [n, k/128]
  const int32_t* offsets; // grouped: [groups + 1]
  void* c;
  int64_t ldc;
  float* cs;              // quantized output: scales [rows, ceil(n/128)]
  bool vec_c;             // ldc % 4 == 0: 16-byte (f32) / 8-byte (bf16) row-fragment stores
  int rows;               // dense: M; grouped: rows_cap; wgrad: Nout
  int n, k, groups;
  int tiles_m, tiles_n;
  int bn;                 // tile width in N: 256, or 224 for the weight gradient (see launch_wgrad)
};

// 16-byte chunk swizzle of a 128-byte LDS row: rows r and r+8 of a 16-row
// fragment also differ, so 16 lanes reading one logical chunk of 16 rows
// cover 16 distinct chunk slots across a pair of rows.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }


// Eight E4M3 codes (two dwords, byte order) -> eight BF16 values, exactly.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(int lo, int hi) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The same with the operand's scale applied by the convert: for a power of
// two 2^e each E4M3 value times 2^e is again a BF16 value (exact), as long as
// it stays in BF16's normal range.
__device__ __forceinline__ v8bf e4m3x8_to_bf16_scaled(int lo, int hi, float s) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, s, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, s, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, s, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, s, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

struct Tile {
  int m0, mend;  // rows [m0, mend) of A / C
  int n0;
  int wrows;     // waves along M: 4 (256-row tile), 2 or 1 (tiles of at most 128 / 64 rows)
  const uint8_t* w;
  const float* sw;
};

// XCD-aware order: workgroup i runs on XCD i % 8, so consecutive logical
// tiles are given to the same XCD (they share L2), grouped 4 tile-rows at a
// time so that one XCD's tiles share A rows and W rows.
__device__ __forceinline__ int xcd_logical(int bid, int nblk) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  return xcd * per + min(xcd, rem) + idx;
}

template <int MODE>
__device__ __forceinline__ bool decode_tile(const GemmArgs& g, Tile& t) {
  const int nkb = g.k / BK;
  if constexpr (MODE == kGrouped) {
    // Grid = (ceil(rows_cap/256) + groups) * tiles_n, an upper bound of the
    // real tile count; workgroups beyond it exit.  N tiles vary fastest, so
    // the XCD of a workgroup fixes its N tiles and W rows stay XCD-local.
    // Tiles are handed out longest first: all tiles of more than 128 rows
    // (every group's full 256-row tiles and long last tiles), then last
    // tiles of 65-128 rows, then those of 1-64 rows, which run on 2 x 4 and
    // 1 x 8 wave layouts and fill in as the long tiles finish.
    const int bid = blockIdx.x;
    const int tn = bid % g.tiles_n;
    int mt = bid / g.tiles_n;
    for (int cls = 0; cls < 3; ++cls) {
      for (int gi = 0; gi < g.groups; ++gi) {
        // a routing table that breaks its precondition (offsets outside
        // [0, rows_cap] or decreasing) is clamped: every tile stays inside
        // the rows of a and c
        const int lo = min(max(g.offsets[gi], 0), g.rows);
        const int hi = min(max(g.offsets[gi + 1], lo), g.rows);
        const int rows = hi - lo;
        const int full = rows / BM, rem = rows % BM;
        const int cnt = cls == 0 ? full + (rem > 128 ? 1 : 0)
                      : cls == 1 ? (rem > 64 && rem <= 128 ? 1 : 0)
                                 : (rem > 0 && rem <= 64 ? 1 : 0);
        if (mt < cnt) {
          t.m0 = lo + (cls == 0 ? mt : full) * BM;
          t.mend = min(t.m0 + BM, hi);
          t.wrows = cls == 0 ? 4 : cls == 1 ? 2 : 1;
          t.n0 = tn * BN;
          t.w = g.w + (int64_t)gi * g.n * g.k;
          t.sw = g.sw + (int64_t)gi * ((g.n + 127) / 128) * nkb;
          return true;
        }
        mt -= cnt;
      }
    }
    return false;
  } else {
    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    const int group = logical / (4 * g.tiles_n);
    const int first = group * 4;
    const int gm = min(g.tiles_m - first, 4);
    const int in = logical - group * 4 * g.tiles_n;
    const int tm = first + in % gm;
    const int tn = in / gm;
    t.m0 = tm * BM;
    t.mend = min(t.m0 + BM, g.rows);
    t.wrows = 4;
    t.n0 = tn * g.bn;
    t.w = g.w;
    t.sw = g.sw;
    return true;
  }
}

// One K block of the main loop.  `cur` (the stage multiplied now) and
// `refill` (the stage the loads of block kb+AHEAD go to) are distinct sets
// of LDS arrays, so the compiler keeps those loads in flight across the LDS
// reads of `cur` instead of waiting for them.  With AHEAD = 1 (two stages)
// the barrier is a bare s_barrier after an explicit vmcnt(0): every wave's
// loads of block kb have landed, and every LDS read of the stage being
// refilled was consumed before its wave got here; __syncthreads() would add
// nothing but a fence.  With AHEAD = 2 (three stages) the wait leaves the
// newest refill in flight.  The asm memory clobber keeps the compiler from
// moving LDS accesses across it.  Past the last block the refill re-reads
// the last block (in bounds) into a stage that is never read again, so the
// issue stays unconditional and the compiler's tracking of the loads in
// flight stays exact.  `compute` calls refill_now() once, at the point where
// the refill loads should go out, after its reads of the scale buffer `scl`
// (the refill of step kb brings a quarter of the next group of four
// blocks' scales into the other half).  A batch of loads starts with its
// scale loads, so waiting for vmcnt(LOADS) (LOADS = the operand loads of
// one batch) also covers batches that carry them.
template <int AHEAD, int LOADS, class Issue, class Compute>
__device__ __forceinline__ void run_step(int kb, int nkb, const uint8_t* __restrict__ cur,
                                         uint8_t* __restrict__ refill, uint8_t* __restrict__ scl, Issue& issue,
                                         Compute& compute) {
  if constexpr (AHEAD == 1) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    // the loads of block kb+1 (issued during block kb-1) may stay in
    // flight; loads complete in order, so block kb's have landed
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LOADS) : "memory");
  }
  auto refill_now = [&]() { issue(min(kb + AHEAD, nkb - 1), refill, scl, kb); };
  compute(cur, scl, kb, refill_now);
}

// The K loops.  Every stage and the scale buffer are __restrict__
// parameters of the one function that runs the whole loop: the compiler's
// tracking of loads in flight into LDS tells them apart only through that
// aliasing information, and it has to hold between a stage's reads and the
// loads into the other stages issued in earlier iterations.
template <int LOADS, class Issue, class Compute>
__device__ __forceinline__ void k_loop2(int nkb, uint8_t* __restrict__ s0, uint8_t* __restrict__ s1,
                                        uint8_t* __restrict__ scl, Issue& issue, Compute& compute) {
  if (nkb > 0) issue(0, s0, scl, -1);
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    run_step<1, LOADS>(kb, nkb, s0, s1, scl, issue, compute);
    run_step<1, LOADS>(kb + 1, nkb, s1, s0, scl, issue, compute);
  }
  if (kb < nkb) run_step<1, LOADS>(kb, nkb, s0, s1, scl, issue, compute);
}

template <int LOADS, class Issue, class Compute>
__device__ __forceinline__ void k_loop3(int nkb, uint8_t* __restrict__ s0, uint8_t* __restrict__ s1,
                                        uint8_t* __restrict__ s2, uint8_t* __restrict__ scl, Issue& issue,
                                        Compute& compute) {
  if (nkb > 0) {
    issue(0, s0, scl, -1);
    issue(min(1, nkb - 1), s1, scl, -2);
  }
  for (int kb = 0; kb < nkb; kb += 3) {
    run_step<2, LOADS>(kb, nkb, s0, s2, scl, issue, compute);
    if (kb + 1 < nkb) run_step<2, LOADS>(kb + 1, nkb, s1, s0, scl, issue, compute);
    if (kb + 2 < nkb) run_step<2, LOADS>(kb + 2, nkb, s2, s1, scl, issue, compute);
  }
}

// NARROW: tiles of 224 columns (dense and weight-gradient launches whose
// column count fills the compute units better that way); a kernel of its
// own, so the 256-column form keeps its registers.
template <int MODE, int OUT, int ACC, int NARROW>
__global__ __launch_bounds__(kThreads) void gemm_bs_kernel(GemmArgs g) {
  // two full stages, or (grouped tiles of at most 128 rows) three small
  // ones, then the scale buffer
  constexpr int kStageBytes = MODE == kGrouped ? 3 * kSmallStage : 2 * kFullStage;
  static_assert(kStageBytes >= 2 * kFullStage, "full tiles of the grouped form use two full stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStageBytes + kSclBytes];

  Tile t;
  if (!decode_tile<MODE>(g, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS addresses
  // waves along M (wave-uniform): 4 x 2 waves of 64 x 128 for a full tile;
  // 2 x 4 of 64 x 64 or 1 x 8 of 64 x 32 for a grouped tile of <= 128 or
  // <= 64 rows
  const int wrows = __builtin_amdgcn_readfirstlane(t.wrows);
  const int wm = wave & (wrows - 1);
  const int wn = wave >> (wrows == 4 ? 2 : wrows == 2 ? 1 : 0);
  const int K = g.k, N = g.n;
  const int nkb = K / BK;

  // ---- global->LDS assignment: one wave instruction moves 8 rows x 128 B.
  // Full tiles: wave w moves rows 32w..32w+31 of both the A and the W tile
  // (into the slot of its 128-row half).  Grouped tiles of at most 128 (64)
  // rows move their A rows as 16 (8) rows per wave and the W tile as full
  // tiles do.  Loads are buffer loads with an LDS destination.  The A buffer
  // covers exactly the tile's rows and the W buffer ends at the operand's
  // last row, so rows past either read as zero (the hardware range check,
  // which also skips the memory access) instead of being clamped.  The
  // K-block offset goes in an SGPR, the LDS address in M0: issuing costs no
  // VALU work.  Offsets fit in 32 bits (the host rejects operands of 2 GiB+).
  const uint32_t rowb = (uint32_t)K;  // bytes per operand row
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + (size_t)t.m0 * rowb), 0, (int)((uint32_t)(t.mend - t.m0) * rowb), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(t.w + (size_t)t.n0 * rowb), 0, (int)((uint32_t)(N - t.n0) * rowb), kRsrcFlags);
  auto row_off = [&](int row) { return (uint32_t)row * rowb + 16u * (uint32_t)((lane & 7) ^ swz(row)); };
  uint32_t r_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r_off[i] = row_off((wave * 4 + i) * 8 + (lane >> 3));
  // scales: waves 0-3 bring the A scales of rows 64w..64w+63, waves 4-7 the
  // W scale of columns 64(w-4)..+63 (one value per column, so all forms
  // share the layout)
  const uint32_t sblk = (uint32_t)nkb * 4u;  // bytes per scale row
  const int sidx = (wave & 3) * 64 + lane;
  __amdgpu_buffer_rsrc_t s_rsrc;
  uint32_t s_off;
  if (wave < 4) {
    s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(g.sa + (size_t)t.m0 * nkb), 0,
                                               (int)((uint32_t)(t.mend - t.m0) * sblk), kRsrcFlags);
    s_off = (uint32_t)sidx * sblk;
  } else if (MODE == kWgrad) {
    s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(t.sw + (size_t)t.n0 * nkb), 0,
                                               (int)((uint32_t)(N - t.n0) * sblk), kRsrcFlags);
    s_off = (uint32_t)sidx * sblk;
  } else {  // one scale row per 128 columns, from the one holding column n0
    s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(t.sw + (size_t)(t.n0 >> 7) * nkb), 0,
                                               (int)((uint32_t)(((N + 127) >> 7) - (t.n0 >> 7)) * sblk), kRsrcFlags);
    s_off = 0;  // (unused: these scales arrive by quarters)
  }
  // Scale buffer fill.  Waves 0-3 own A rows 64w..64w+63, waves 4-7 W
  // columns 64(w-4)..+63, laid out [entry][4 blocks] in each half.  One
  // 4-byte load instruction covers 16 entries x 4 blocks (lane i: entry i/4,
  // block i%4), so the step kb refill brings quarter kb%4 of group kb/4+1
  // into half (kb/4+1)%2, whose last reader (group kb/4-1) is behind the
  // barrier of this step; group g is complete when step 4g begins.  The
  // prologue (step -1) brings group 0 whole; step -2 (the second prologue
  // batch of three stages) brings none.  Every offset is in the VGPR part, so
  // the buffer's range check turns entries past the tile and blocks past
  // k/128 into zeros.  The weight gradient's W scales (per column and block)
  // go into the block's stage instead, one block per load.  Issued first in
  // a batch.
  // (the dense and grouped W entries are columns: column e of the tile reads
  // the scale row of its 128-column block, ((n0 mod 128) + e) / 128 rows past
  // the buffer's first)
  const int q_entry = (wave & 3) * 64 + (lane >> 2);  // entry of quarter 0
  const bool row_entries = MODE == kWgrad || wave < 4;
  const uint32_t q_lane = 4u * (uint32_t)(lane & 3);
  // (grouped tiles start at a multiple of 256 columns: a W wave's 64
  // columns share one scale row)
  const uint32_t q_voff = (row_entries ? (uint32_t)q_entry : (uint32_t)((wave & 3) >> 1)) * sblk + q_lane;
  auto scale_quarter = [&](uint8_t* scl, int grp, int qq) {
    uint8_t* half = scl + (grp & 1) * kSclHalf + (wave < 4 ? 0 : BM * 16) + ((wave & 3) * 64 + 16 * qq) * 16;
    uint32_t off;
    if (MODE == kDense && !row_entries) {
      off = (uint32_t)(((t.n0 & 127) + q_entry + 16 * qq) >> 7) * sblk + q_lane;
    } else {
      off = q_voff + (row_entries ? (uint32_t)(16 * qq) * sblk : 0u);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_void_ptr)half, 4, off + (uint32_t)grp * 16u, 0, 0, 0);
  };
  auto issue_scales = [&](int kb, uint8_t* st, uint8_t* scl, int step) {
    if (MODE == kWgrad && wave >= 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_void_ptr)(st + StageLayout<BM>::kS + (wave & 3) * 256), 4,
                                               s_off, (uint32_t)kb * 4u, 0, 0);
    } else if (step >= 0) {
      scale_quarter(scl, (step >> 2) + 1, step & 3);
    } else if (step == -1) {
      scale_quarter(scl, 0, 0);
      scale_quarter(scl, 0, 1);
      scale_quarter(scl, 0, 2);
      scale_quarter(scl, 0, 3);
    }
  };

  // full tile: the scale load, then 4 A + 4 W loads per wave
  auto issue_full = [&](int kb, uint8_t* st, uint8_t* scl, int step) {
    using L = StageLayout<BM>;
    issue_scales(kb, st, scl, step);
    const uint32_t kofs = (uint32_t)kb * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(st + (wave * 4 + i) * 1024), 16, r_off[i], kofs, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(st + L::kW + (wave * 4 + i) * 1024), 16, r_off[i], kofs, 0, 0);
    }
  };

  v4f acc[4][8];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  bool active = false;  // set per wave layout below
  const int r16 = lane & 15;
  const int c0 = 2 * (lane >> 4);
  // a stage's layout for the wave layout of JN 16-column W fragments per
  // wave (JN = 8: full tile; 4: at most 128 rows; 2: at most 64 rows)
  auto layout_of = [](auto jn) {
    constexpr int JN = decltype(jn)::value;
    return StageLayout<JN >= 7 ? BM : JN == 4 ? 128 : 64>{};
  };

  // One K block: 8 W fragments (j) x 4 M fragments (f) x 4 K steps of 32 (q)
  // = 128 MFMAs per wave.  Explicit software pipeline, in program order:
  //   - the block's A fragments and W fragment 0 are read first and widened
  //     during j = 0, each q-part right before its MFMA group;
  //   - W fragment j+1 is widened to BF16 during j, q-part by q-part, each
  //     into the slot whose MFMAs have all been issued; each half of its
  //     E4M3 bytes, once widened, is refilled from LDS with fragment j+2's,
  //     three MFMA groups ahead of use;
  //   - the four partial chains (f) are interleaved, so an MFMA never waits
  //     for the one it accumulates onto;
  //   - the fold of fragment j's partial for M fragment f is placed right
  //     before the first MFMA of fragment j+1 that overwrites it, 4 MFMAs
  //     after its last one.
  // sched_barrier(0) keeps the compiler from regrouping the MFMAs.
  auto compute_bf16 = [&](const uint8_t* st, const float* SA, auto& refill_now, auto jn) {
    constexpr int JN = decltype(jn)::value;  // 16-column W fragments per wave
    constexpr int WC = 16 * JN;
    if (!active) {
      refill_now();
      return;
    }
    using L = decltype(layout_of(jn));
    const float* S = reinterpret_cast<const float*>(st + L::kS);
    float sa[4];
    const int arow0 = wm * 64 + r16;
#pragma unroll
    for (int f = 0; f < 4; ++f) sa[f] = SA[(arow0 + f * 16) * 4];
    // Fold scales.  A wave's columns lie in one 128-column block except in
    // dense tiles of 224 columns (JN = 7), whose 112 columns per wave may
    // reach into a second block: fragments j < jb (16 columns each, inside
    // one block) take the first block's weight scale, the others the
    // second's (sc2).
    constexpr bool kFragScale = MODE == kDense && JN != 8;
    float sc[4], sc2[4];
    const int jb = kFragScale ? (128 - ((t.n0 + wn * WC) & 127)) >> 4 : JN;
    if constexpr (MODE != kWgrad) {
      const float swv = SA[(BM + wn * WC) * 4];
      const float swv2 = kFragScale ? SA[(BM + wn * WC + WC - 16) * 4] : 0.f;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        sc[f] = sa[f] * swv;
        if constexpr (kFragScale) sc2[f] = sa[f] * swv2;
      }
    }
    // Wgrad issues the refill later (see below); the other forms once the
    // scales are read
    if (MODE != kWgrad) refill_now();
    const int wrow0 = wn * WC + r16;
    const int wsw = swz(wrow0);  // same swizzle for rows wrow0 + 16j
    // one base address per half; fragment j is 2 KiB further (an
    // immediate offset of the LDS read)
    const uint8_t* Wb = st + L::kW + wrow0 * 128;
    const uint8_t* w_lo = Wb + 16 * (c0 ^ wsw);
    const uint8_t* w_hi = Wb + 16 * ((c0 + 1) ^ wsw);
    auto read_w_lo = [&](int j, v4i& lo) { lo = *reinterpret_cast<const v4i*>(w_lo + j * 2048); };
    auto read_w_hi = [&](int j, v4i& hi) { hi = *reinterpret_cast<const v4i*>(w_hi + j * 2048); };
    auto part = [](const v4i& lo, const v4i& hi, int q) {
      const v4i& r = q < 2 ? lo : hi;
      return e4m3x8_to_bf16(r[(q & 1) * 2], r[(q & 1) * 2 + 1]);
    };
    const int asw = swz(arow0);  // same swizzle for rows arow0 + 16f
    // A fragments and W fragment 0 are widened q-part by q-part during
    // j = 0, each right before the MFMA group that first needs it, so the
    // block does not open with a burst of 80 converts and no MFMA (5%
    // faster than widening them up front)
    v8bf af[4][4];  // A fragments widened to BF16: [f][q]
    v4i alo[4], ahi[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint8_t* base = st + (arow0 + f * 16) * 128;
      alo[f] = *reinterpret_cast<const v4i*>(base + 16 * (c0 ^ asw));
      ahi[f] = *reinterpret_cast<const v4i*>(base + 16 * ((c0 + 1) ^ asw));
    }
    v4i w0lo, w0hi;  // E4M3 bytes of W fragment 0
    v4i wlo, whi;    // E4M3 bytes of the next W fragment
    v8bf bf[4];      // the current W fragment widened to BF16: [q]
    read_w_lo(0, w0lo);
    read_w_hi(0, w0hi);
    if constexpr (MODE == kWgrad) {
      // the Wgrad fold holds more registers: widen up front so the raw
      // bytes die before the MFMAs start (no spills)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf[q] = part(w0lo, w0hi, q);
#pragma unroll
        for (int f = 0; f < 4; ++f) af[f][q] = part(alo[f], ahi[f], q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    read_w_lo(1, wlo);
    read_w_hi(1, whi);
    v4f p[4];
    // Wgrad: the column scales of fragment j, read once during j (after its
    // first MFMA group, when fragment j-1's folds are done) and used by j's
    // folds.  Their address is formed from the per-lane thread index so it
    // stays one register plus an immediate per fragment (with the
    // wave-uniform index the compiler keeps one register per fragment and
    // stage, which spilled).
    const int wn_lane = (tid >> 6) >> (wrows == 4 ? 2 : wrows == 2 ? 1 : 0);
    const float* swp = S + wn_lane * WC + 4 * (lane >> 4);
    v4f swj = v4f{0.f, 0.f, 0.f, 0.f};
    auto fold = [&](int j, int f) {
      if constexpr (MODE == kWgrad) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][j][v] = __builtin_fmaf(p[f][v], sa[f] * swj[v], acc[f][j][v]);
      } else {
        const float s = kFragScale && j >= jb ? sc2[f] : sc[f];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][j][v] = __builtin_fmaf(p[f][v], s, acc[f][j][v]);
      }
    };

#pragma unroll
    for (int j = 0; j < JN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j == 0 && MODE != kWgrad) {
          bf[q] = part(w0lo, w0hi, q);
#pragma unroll
          for (int f = 0; f < 4; ++f) af[f][q] = part(alo[f], ahi[f], q);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (q == 0 && j > 0) fold(j - 1, f);
          p[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[q], af[f][q],
                                                          q == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : p[f], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Wgrad (its fold keeps more values live and the compiler spills a
        // few prologue values) issues the refill of the other stage once the
        // block's first fragments are in registers: a register reload after
        // the refill would wait for it (measured 693 -> 460 us for
        // 2048 x 7168 over 16384 tokens; the dense form is 5% slower so)
        if (MODE == kWgrad && j == 0 && q == 0) refill_now();
        // slot q is no longer needed by fragment j: widen fragment j+1's part
        if (j < JN - 1) bf[q] = part(wlo, whi, q);
        if constexpr (MODE == kWgrad) {
          if (q == 0) swj = *reinterpret_cast<const v4f*>(swp + j * 16);
        }
        // a consumed half of fragment j+1's bytes is refilled with fragment
        // j+2's right away: three MFMA groups before it is needed
        if (q == 1 && j < JN - 2) read_w_lo(j + 2, wlo);
        if (q == 3 && j < JN - 2) read_w_hi(j + 2, whi);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) fold(JN - 1, f);
  };

  // Float32-grade form for power-of-two scales: each fragment is widened
  // with its operand's scale applied by the convert (exact, see
  // e4m3x8_to_bf16_scaled), so every product is sa*sw*a*w and all K blocks
  // chain onto the same matrix-core accumulator: no fold.  The scales of a
  // block are read before its refill (as in the FP32-grade form); the
  // dense and grouped W scale of a column is its 128-column block's, the
  // weight gradient's its own (in the stage).
  auto compute_bf16s = [&](const uint8_t* st, const float* SA, auto& refill_now, auto jn) {
    constexpr int JN = decltype(jn)::value;  // 16-column W fragments per wave
    constexpr int WC = 16 * JN;
    if (!active) {
      refill_now();
      return;
    }
    using L = decltype(layout_of(jn));
    const float* S = reinterpret_cast<const float*>(st + L::kS);
    const int arow0 = wm * 64 + r16;
    const int wrow0 = wn * WC + r16;
    float sa[4], sw[JN];
#pragma unroll
    for (int f = 0; f < 4; ++f) sa[f] = SA[(arow0 + f * 16) * 4];
#pragma unroll
    for (int j = 0; j < JN; ++j) sw[j] = MODE == kWgrad ? S[wrow0 + j * 16] : SA[(BM + wrow0 + j * 16) * 4];
    refill_now();
    const int wsw = swz(wrow0);
    const uint8_t* Wb = st + L::kW + wrow0 * 128;
    const uint8_t* w_lo = Wb + 16 * (c0 ^ wsw);
    const uint8_t* w_hi = Wb + 16 * ((c0 + 1) ^ wsw);
    auto read_w_lo = [&](int j, v4i& lo) { lo = *reinterpret_cast<const v4i*>(w_lo + j * 2048); };
    auto read_w_hi = [&](int j, v4i& hi) { hi = *reinterpret_cast<const v4i*>(w_hi + j * 2048); };
    auto part = [](const v4i& lo, const v4i& hi, int q, float sc) {
      const v4i& r = q < 2 ? lo : hi;
      return e4m3x8_to_bf16_scaled(r[(q & 1) * 2], r[(q & 1) * 2 + 1], sc);
    };
    const int asw = swz(arow0);
    v8bf af[4][4];
    v4i alo[4], ahi[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint8_t* base = st + (arow0 + f * 16) * 128;
      alo[f] = *reinterpret_cast<const v4i*>(base + 16 * (c0 ^ asw));
      ahi[f] = *reinterpret_cast<const v4i*>(base + 16 * ((c0 + 1) ^ asw));
    }
    v4i w0lo, w0hi, wlo, whi;
    v8bf bf[4];
    read_w_lo(0, w0lo);
    read_w_hi(0, w0hi);
    read_w_lo(1, wlo);
    read_w_hi(1, whi);
#pragma unroll
    for (int j = 0; j < JN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j == 0) {
          bf[q] = part(w0lo, w0hi, q, sw[0]);
#pragma unroll
          for (int f = 0; f < 4; ++f) af[f][q] = part(alo[f], ahi[f], q, sa[f]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[q], af[f][q], acc[f][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j < JN - 1) bf[q] = part(wlo, whi, q, sw[j + 1]);
        if (q == 1 && j < JN - 2) read_w_lo(j + 2, wlo);
        if (q == 3 && j < JN - 2) read_w_hi(j + 2, whi);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // FP8 matrix-core form: one v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile
  // and K block reads the E4M3 bytes straight from LDS (lane group g holds
  // bytes 32g..32g+31 of its row, the instruction's operand layout).  Its
  // partial is formed inside the matrix core at the precision measured for
  // it (groups of 8 consecutive products aligned to the group's largest one
  // and truncated about 14 bits below it), which is the pages' limited
  // in-core accumulation; the fold into FP32 every 128 elements is the same.
  // Per K block: the fragments are read first (W fragment 0, then the four
  // A fragments, then the scales), the refill of the other stage goes out
  // after the first MFMA group, and W fragment j+1 is read while j runs.
  auto compute_f8 = [&](const uint8_t* st, const float* SA, auto& refill_now, auto jn) {
    constexpr int JN = decltype(jn)::value;
    constexpr int WC = 16 * JN;
    if (!active) {
      refill_now();
      return;
    }
    using L = decltype(layout_of(jn));
    const float* S = reinterpret_cast<const float*>(st + L::kS);
    const int wrow0 = wn * WC + r16;
    const uint8_t* Wb = st + L::kW + wrow0 * 128;
    const uint8_t* Ab = st + (wm * 64 + r16) * 128;
    const int wsw = swz(wrow0);
    const int arow0 = wm * 64 + r16;
    const int asw = swz(arow0);
    auto read8 = [&](const uint8_t* rowp, int sw) {
      const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c0 ^ sw));
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * ((c0 + 1) ^ sw));
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    v8i wf[2];
    wf[0] = read8(Wb, wsw);
    v8i af[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) af[f] = read8(Ab + f * 16 * 128, asw);
    float sa[4], sc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) sa[f] = SA[(arow0 + f * 16) * 4];
    // (dense tiles of 224 columns: fragments j >= jb take the second
    // block's weight scale, as in the BF16 form)
    constexpr bool kFragScale = MODE == kDense && JN != 8;
    float sc2[4];
    const int jb = kFragScale ? (128 - ((t.n0 + wn * WC) & 127)) >> 4 : JN;
    const float swv = SA[(BM + wn * WC) * 4];
    const float swv2 = kFragScale ? SA[(BM + wn * WC + WC - 16) * 4] : 0.f;
    __builtin_amdgcn_sched_barrier(0);
    v4f p[4];
    // Wgrad: column scales of the fragment being folded, read once per
    // fragment (after the previous fragment's folds) instead of per fold
    const float* swp = S + wn * WC + 4 * (lane >> 4);
    v4f swj = v4f{0.f, 0.f, 0.f, 0.f};
    auto fold = [&](int j, int f) {
      if constexpr (MODE == kWgrad) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][j][v] = __builtin_fmaf(p[f][v], sa[f] * swj[v], acc[f][j][v]);
      } else {
        const float s = kFragScale && j >= jb ? sc2[f] : sc[f];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][j][v] = __builtin_fmaf(p[f][v], s, acc[f][j][v]);
      }
    };
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      if (j < JN - 1) wf[(j + 1) & 1] = read8(Wb + (j + 1) * 16 * 128, wsw);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (j > 0) fold(j - 1, f);
        p[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j & 1], af[f], v4f{0.f, 0.f, 0.f, 0.f},
                                                               0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MODE == kWgrad) swj = *reinterpret_cast<const v4f*>(swp + j * 16);
      if (j == 0) {
        refill_now();
        if constexpr (MODE != kWgrad) {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            sc[f] = sa[f] * swv;
            if constexpr (kFragScale) sc2[f] = sa[f] * swv2;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) fold(JN - 1, f);
  };

  // Hardware-scaled form (power-of-two scales only): the E8M0 exponent of
  // each operand row's scale rides along with v_mfma_scale_f32_16x16x128_f8f6f4,
  // which applies it inside the matrix core, and every K block accumulates
  // into the same matrix-core accumulator -- the pages' "MMA with group
  // scaling" (tmdrlife.com wr_id=13334 ¶3) and, with it, no promotion: the
  // running sum never leaves the unit until the epilogue.
  auto compute_f8s = [&](const uint8_t* st, const float* SA, auto& refill_now, auto jn) {
    constexpr int JN = decltype(jn)::value;
    constexpr int WC = 16 * JN;
    if (!active) {
      refill_now();
      return;
    }
    using L = decltype(layout_of(jn));
    const int wrow0 = wn * WC + r16;
    const uint8_t* Wb = st + L::kW + wrow0 * 128;
    const uint8_t* Ab = st + (wm * 64 + r16) * 128;
    const int wsw = swz(wrow0);
    const int arow0 = wm * 64 + r16;
    const int asw = swz(arow0);
    auto read8 = [&](const uint8_t* rowp, int sw) {
      const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c0 ^ sw));
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * ((c0 + 1) ^ sw));
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto e8m0 = [](float x) { return (int)((__float_as_uint(x) >> 23) & 0xFFu); };
    v8i wf[2];
    wf[0] = read8(Wb, wsw);
    v8i af[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) af[f] = read8(Ab + f * 16 * 128, asw);
    // every scale of the block is read before the refill goes out (it may
    // write the other half of the scale buffer); the weight gradient's W
    // scales (per column and block) are in the stage
    const float* SS = reinterpret_cast<const float*>(st + L::kS);
    int ae[4], we[JN];
#pragma unroll
    for (int f = 0; f < 4; ++f) ae[f] = e8m0(SA[(arow0 + f * 16) * 4]);
#pragma unroll
    for (int j = 0; j < JN; ++j)  // this lane's W row
      we[j] = e8m0(MODE == kWgrad ? SS[wrow0 + j * 16] : SA[(BM + wrow0 + j * 16) * 4]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      if (j < JN - 1) wf[(j + 1) & 1] = read8(Wb + (j + 1) * 16 * 128, wsw);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        acc[f][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j & 1], af[f], acc[f][j], 0, 0,
                                                                     0, we[j], 0, ae[f]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        refill_now();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto compute = [&](const uint8_t* st, const uint8_t* scl, int kb, auto& refill_now, auto jn) {
    // this block's scales in the scale buffer: A entry e at SA[4 e], W
    // entry e at SA[4 (BM + e)]
    const float* SA = reinterpret_cast<const float*>(scl + ((kb >> 2) & 1) * kSclHalf) + (kb & 3);
    if constexpr (ACC == 3) {
      compute_bf16s(st, SA, refill_now, jn);
    } else if constexpr (ACC == 2) {
      compute_f8s(st, SA, refill_now, jn);
    } else if constexpr (ACC == 1) {
      compute_f8(st, SA, refill_now, jn);
    } else {
      compute_bf16(st, SA, refill_now, jn);
    }
  };

  auto run = [&](auto jn) {
    constexpr int JN = decltype(jn)::value;
    constexpr int WC = 16 * JN;
    active = (wm * 64 < t.mend - t.m0) && (wn * WC < N - t.n0);
    auto comp = [&](const uint8_t* st, const uint8_t* scl, int kb, auto& refill_now) {
      compute(st, scl, kb, refill_now, jn);
    };
    if constexpr (MODE == kGrouped && JN < 8) {
      // A grouped tile of at most 128 (JN = 4) or 64 (JN = 2) rows does a
      // fraction of a full tile's arithmetic per K block but streams the
      // same 256 weight rows, so it is bound by the latency of its loads:
      // three stages keep two K blocks in flight.  Its A rows are moved as
      // 16 (8) rows per wave, the weight rows as in a full tile.
      // (the A row offsets are spelled out instead of looping over a local
      // constant inside the lambda: that form leaves the host compiler
      // without the kernel's launch stub)
      const uint32_t ra_off0 = row_off((JN == 4 ? wave * 2 : wave) * 8 + (lane >> 3));
      const uint32_t ra_off1 = row_off((wave * 2 + 1) * 8 + (lane >> 3));
      using L = decltype(layout_of(jn));
      auto issue_small = [&](int kb, uint8_t* st, uint8_t* scl, int step) {
        issue_scales(kb, st, scl, step);
        const uint32_t kofs = (uint32_t)kb * BK;
        if constexpr (decltype(jn)::value == 4) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(st + (wave * 2) * 1024), 16, ra_off0,
                                                   kofs, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(st + (wave * 2 + 1) * 1024), 16, ra_off1,
                                                   kofs, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(st + wave * 1024), 16, ra_off0, kofs, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(st + L::kW + (wave * 4 + i) * 1024), 16,
                                                   r_off[i], kofs, 0, 0);
      };
      k_loop3<(JN == 4 ? 2 : 1) + 4>(nkb, lds, lds + kSmallStage, lds + 2 * kSmallStage, lds + kStageBytes,
                                     issue_small, comp);
    } else {
      // Two full stages: block kb+1 streams in while kb is multiplied.
      k_loop2<8>(nkb, lds, lds + kFullStage, lds + kStageBytes, issue_full, comp);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: lane holds C[m][n..n+3]
    if constexpr (OUT == kOutE4M3 || OUT == kOutE4M3Pow2) {
      // The BF16 value of each output, quantized per 1x128 tile along N:
      // the wave's 128 columns are one tile (dense: WC = 128 and n0 a
      // multiple of 256), held by the four lanes that share r16, 32 values
      // each.  Tile max-abs over BF16 magnitude bits, reduced across those
      // lanes with every lane of the wave active; the scale and the codes
      // then come from the 1x128 quantizer's own helpers.
      static_assert(WC == 128, "one 1x128 tile per wave and row");
      constexpr bool P2 = OUT == kOutE4M3Pow2;
      const int nbc = (N + 127) >> 7;
      const int tn0 = t.n0 + wn * WC;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int m = t.m0 + wm * 64 + f * 16 + r16;
        uint32_t bits[JN][4];
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < JN; ++j) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = tn0 + j * 16 + 4 * (lane >> 4) + v;
            bits[j][v] = n < N ? bf16_rne_bits(acc[f][j][v]) : 0u;
            amax = max(amax, bits[j][v] & 0x7FFFu);
          }
        }
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 16));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
        const TileScale ts = tile_scale<P2>(amax);
        uint8_t* crow = reinterpret_cast<uint8_t*>(g.c) + (int64_t)m * g.ldc;
        with_quotient<P2>(ts, [&](auto q) {
          if (m >= t.mend) return;
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int n = tn0 + j * 16 + 4 * (lane >> 4);
            const uint32_t c4 = pack4_e4m3(q(__uint_as_float(bits[j][0] << 16)), q(__uint_as_float(bits[j][1] << 16)),
                                           q(__uint_as_float(bits[j][2] << 16)), q(__uint_as_float(bits[j][3] << 16)));
            if (n + 3 < N && g.vec_c) {
              *reinterpret_cast<uint32_t*>(crow + n) = c4;
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v)
                if (n + v < N) crow[n + v] = (uint8_t)(c4 >> (8 * v));
            }
          }
          if ((lane >> 4) == 0 && tn0 < N) g.cs[(int64_t)m * nbc + (tn0 >> 7)] = ts.s;
        });
      }
    } else {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int m = t.m0 + wm * 64 + f * 16 + r16;
      if (m >= t.mend) continue;
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int n = t.n0 + wn * WC + j * 16 + 4 * (lane >> 4);
        const v4f r = acc[f][j];
        if constexpr (OUT == kOutBF16) {
          uint16_t* crow = reinterpret_cast<uint16_t*>(g.c) + (int64_t)m * g.ldc;
          if (n + 3 < N && g.vec_c) {
            uint2 pk;
            pk.x = bf16_rne_bits(r[0]) | (bf16_rne_bits(r[1]) << 16);
            pk.y = bf16_rne_bits(r[2]) | (bf16_rne_bits(r[3]) << 16);
            *reinterpret_cast<uint2*>(crow + n) = pk;
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (n + v < N) crow[n + v] = (uint16_t)bf16_rne_bits(r[v]);
          }
        } else {
          float* crow = reinterpret_cast<float*>(g.c) + (int64_t)m * g.ldc;
          if (n + 3 < N && g.vec_c) {
            *reinterpret_cast<v4f*>(crow + n) = r;
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (n + v < N) crow[n + v] = r[v];
          }
        }
      }
    }
    }
  };
  if constexpr (MODE == kGrouped) {
    if (wrows == 4) {
      run(std::integral_constant<int, 8>{});
    } else if (wrows == 2) {
      run(std::integral_constant<int, 4>{});
    } else {
      run(std::integral_constant<int, 2>{});
    }
  } else if constexpr (NARROW) {
    // 224-column tiles: the waves split them as 2 x 112 columns (7 W
    // fragments each); the stage still receives 256 W rows (the last 32
    // belong to the next tile and are not used)
    static_assert(MODE == kWgrad || (MODE == kDense && (OUT == kOutF32 || OUT == kOutBF16)),
                  "224-column tiles: dense (float32 / BF16 out) and weight-gradient forms");
    run(std::integral_constant<int, 7>{});
  } else {
    run(std::integral_constant<int, 8>{});
  }
}

// Tile width in N for a dense or weight-gradient launch.  One tile per CU
// and round of tiles, so the time goes as (rounds of tiles) x (tile width);
// 224 columns when that is smaller.  The 2048 x 7168 weight gradient has 224
// tiles of 256 columns, which leave 32 of 256 CUs idle, or 256 of 224, which
// fill them; the 4096 x 7168 Dgrad has 448 tiles of 256 (1.75 rounds, two
// rounds of 256 columns) or 512 of 224 (two rounds of 224 columns).
int tile_width(int tiles_m, int n) {
  const int64_t cus = device_cus();
  auto cost = [&](int bn) {
    const int64_t tiles = (int64_t)tiles_m * ((n + bn - 1) / bn);
    return ((tiles + cus - 1) / cus) * bn;
  };
  return cost(224) < cost(BN) ? 224 : BN;
}

template <int MODE, int OUT, int NARROW>
void launch_acc_w(const GemmArgs& g, int grid, int acc, hipStream_t stream) {
  if (acc == 3) {
    hipLaunchKernelGGL((gemm_bs_kernel<MODE, OUT, 3, NARROW>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else if (acc == 2) {
    hipLaunchKernelGGL((gemm_bs_kernel<MODE, OUT, 2, NARROW>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else if (acc == 1) {
    hipLaunchKernelGGL((gemm_bs_kernel<MODE, OUT, 1, NARROW>), dim3(grid), dim3(kThreads), 0, stream, g);
  } else {
    hipLaunchKernelGGL((gemm_bs_kernel<MODE, OUT, 0, NARROW>), dim3(grid), dim3(kThreads), 0, stream, g);
  }
}

template <int MODE, int OUT>
hipError_t launch_acc(const GemmArgs& g, int grid, int acc, hipStream_t stream) {
  if constexpr (MODE == kWgrad || (MODE == kDense && (OUT == kOutF32 || OUT == kOutBF16))) {
    if (g.bn == 224) {
      launch_acc_w<MODE, OUT, 1>(g, grid, acc, stream);
      return hipGetLastError();
    }
  }
  launch_acc_w<MODE, OUT, 0>(g, grid, acc, stream);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < kMaxDevices) {
    if (const int c = cache[dev].load(std::memory_order_relaxed)) return c;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Outputs up to which the dense float32-grade GEMM runs the 32 x 32 split-K
// kernel (-1: the default, 8192 per compute unit, i.e. as many outputs as
// an eighth of the compute units hold in 256 x 256 tiles).
namespace {
std::atomic<int64_t> g_small_limit{-1};
}

int64_t small_gemm_limit() {
  const int64_t v = g_small_limit.load(std::memory_order_relaxed);
  return v >= 0 ? v : (int64_t)device_cus() * 8192;
}

int64_t set_small_gemm_limit(int64_t max_outputs) {
  return g_small_limit.exchange(max_outputs < 0 ? -1 : max_outputs, std::memory_order_relaxed);
}

hipError_t launch_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                       const float* w_scales, int m, int n, int k, bool bf16_out, int acc,
                       void* c, int64_t ldc, hipStream_t stream) {
  if (acc == 0 && (int64_t)m * n <= small_gemm_limit())
    return launch_gemm_small(a, a_scales, w, w_scales, m, n, k, bf16_out, c, ldc, stream);
  GemmArgs g{};
  g.a = a; g.sa = a_scales; g.w = w; g.sw = w_scales; g.offsets = nullptr;
  g.c = c; g.ldc = ldc; g.vec_c = (ldc % 4) == 0; g.rows = m; g.n = n; g.k = k; g.groups = 1;
  g.tiles_m = (m + BM - 1) / BM;
  g.bn = tile_width(g.tiles_m, n);
  g.tiles_n = (n + g.bn - 1) / g.bn;
  const int grid = g.tiles_m * g.tiles_n;
  return bf16_out ? launch_acc<kDense, kOutBF16>(g, grid, acc, stream)
                  : launch_acc<kDense, kOutF32>(g, grid, acc, stream);
}

hipError_t launch_gemm_quantized(const uint8_t* a, const float* a_scales, const uint8_t* w,
                                 const float* w_scales, int m, int n, int k, int acc, bool pow2,
                                 uint8_t* codes, int64_t ldc, float* scales, hipStream_t stream) {
  GemmArgs g{};
  g.a = a; g.sa = a_scales; g.w = w; g.sw = w_scales; g.offsets = nullptr;
  g.c = codes; g.ldc = ldc; g.cs = scales; g.vec_c = (ldc % 4) == 0; g.rows = m; g.n = n; g.k = k; g.groups = 1;
  g.tiles_m = (m + BM - 1) / BM;
  g.tiles_n = (n + BN - 1) / BN;
  g.bn = BN;
  const int grid = g.tiles_m * g.tiles_n;
  return pow2 ? launch_acc<kDense, kOutE4M3Pow2>(g, grid, acc, stream)
              : launch_acc<kDense, kOutE4M3>(g, grid, acc, stream);
}

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_scales, const int32_t* offsets,
                               int groups, int rows_cap, const uint8_t* w, const float* w_scales,
                               int n, int k, bool bf16_out, int acc, void* c, int64_t ldc,
                               hipStream_t stream) {
  GemmArgs g{};
  g.a = a; g.sa = a_scales; g.w = w; g.sw = w_scales; g.offsets = offsets;
  g.c = c; g.ldc = ldc; g.vec_c = (ldc % 4) == 0; g.rows = rows_cap; g.n = n; g.k = k; g.groups = groups;
  g.tiles_m = (rows_cap + BM - 1) / BM + groups;  // upper bound of m tiles over all groups
  g.tiles_n = (n + BN - 1) / BN;
  g.bn = BN;
  const int grid = g.tiles_m * g.tiles_n;
  return bf16_out ? launch_acc<kGrouped, kOutBF16>(g, grid, acc, stream)
                  : launch_acc<kGrouped, kOutF32>(g, grid, acc, stream);
}

hipError_t launch_wgrad(const uint8_t* dy_t, const float* dy_scales, const uint8_t* x_t,
                        const float* x_scales, int nout, int kin, int t, int acc, float* dw,
                        int64_t lddw, hipStream_t stream) {
  GemmArgs g{};
  g.a = dy_t; g.sa = dy_scales; g.w = x_t; g.sw = x_scales; g.offsets = nullptr;
  g.c = dw; g.ldc = lddw; g.vec_c = (lddw % 4) == 0; g.rows = nout; g.n = kin; g.k = t; g.groups = 1;
  g.tiles_m = (nout + BM - 1) / BM;
  g.bn = tile_width(g.tiles_m, kin);
  g.tiles_n = (kin + g.bn - 1) / g.bn;
  return launch_acc<kWgrad, kOutF32>(g, g.tiles_m * g.tiles_n, acc, stream);
}

}  // namespace fp8q
