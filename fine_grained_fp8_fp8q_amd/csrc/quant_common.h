// Device helpers for the online max-abs E4M3 quantizers (gfx950).
//
// Tile scale and element code (jp-study.kr doc 258368 ¶1; tmdrlife.com
// wr_id=13334 ¶4):
//   free:  s = RN32(amax / 448), code = E4M3_RNE(RN32(x / s))
//   pow2:  s = smallest 2^e with amax / s <= 448, code = E4M3_RNE(x / s) (exact quotient)
//   amax = 0: s = 0, codes are the signed zeros of the inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8q {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16-byte load and 8/16-byte stores: each byte is
// touched once, so nothing is worth keeping in the caches.
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream8(void* p, uint2 c) {
  __builtin_nontemporal_store(u32x2{c.x, c.y}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_stream16(void* p, uint4 c) {
  __builtin_nontemporal_store(u32x4{c.x, c.y, c.z, c.w}, reinterpret_cast<u32x4*>(p));
}

// Packed 16-bit unsigned max.  BF16 magnitudes (bits & 0x7FFF) order like
// unsigned integers for finite values, so the tile max-abs is an integer max.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  u16x2 x = __builtin_bit_cast(u16x2, a);
  u16x2 y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Max-abs BF16 pattern of the 8 values in a 16-byte chunk (as 0..0x7FFF).
__device__ __forceinline__ uint32_t absmax8(uint4 v) {
  const uint32_t k = 0x7FFF7FFFu;
  uint32_t m = pk_max_u16(pk_max_u16(v.x & k, v.y & k), pk_max_u16(v.z & k, v.w & k));
  return max(m & 0xFFFFu, m >> 16);
}

// Max over the 16 lanes of a DPP row (lanes 16r..16r+15): xor-1 and xor-2
// quad permutes, then half-row and row mirrors.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t dpp_max16(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// float32 -> BF16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four float32 values -> four E4M3 codes (bytes in argument order) with the
// hardware convert, round-to-nearest-even.  Inputs never exceed 448 by more
// than a float32 rounding, which still rounds to 448.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// Per-tile scale state.  For free scales, `mul` = RN32(1/s) and the quotient
// is RN32(x/s) computed with one Markstein correction (M. Markstein, IBM J.
// Res. Dev. 34(1), 1990): q0 = x*r, e = fma(-q0, s, x), q = fma(e, r, q0).
// For BF16 x and amax >= 2^-90 this equals the IEEE quotient for every pair
// whose quotient is >= 2^-10 (smaller quotients encode to zero either way).
// A tile with a smaller (nonzero) amax scales x and s by 2^64 first (exact;
// x' / s' = x / s), and the same three steps on (x', s') equal the IEEE
// quotient for every such pair.  Both claims are checked on the host over
// every BF16 (x, amax) pair.  For power-of-two scales the quotient is an
// exact ldexp.
struct TileScale {
  float s;       // the scale written out (0 for an all-zero tile)
  float div;     // divisor used for the quotient: s, s * 2^64 for a tiny tile, 1 for a zero tile
  float mul;     // RN32(1 / div)
  float xscale;  // x is multiplied by this first: 2^64 for a tiny tile, else 1
  int neg_e;     // pow2: -e
  bool slow;     // free scales with a tiny amax: x and s scaled by 2^64
};

constexpr uint32_t kMarksteinMinAmaxBits = 37u << 7;  // BF16 pattern of 2^-90

// The scale and the reciprocal of the divisor take no IEEE division either:
// s = RN32(amax / 448) is the same Markstein correction of amax * RN32(1/448),
// and RN32(1 / div) is one Newton step, fma(fma(-div, y, 1), y, y), from the
// hardware reciprocal y.  For every nonzero finite BF16 amax the first equals
// the IEEE quotient, and the second equals the IEEE reciprocal of each
// divisor a tile can have (s, or s * 2^64 for a tiny amax) from every y
// within 2 ulps of it (the hardware's is documented within 1); both are
// checked on the host over all 32,639 such amax.
__device__ __forceinline__ TileScale tile_scale_free(uint32_t amax_bits) {
  TileScale t;
  const float amax = __uint_as_float(amax_bits << 16);
  constexpr float kInv448 = 1.0f / 448.0f;  // RN32(1/448)
  const float q0 = amax * kInv448;
  const float s = __builtin_fmaf(__builtin_fmaf(-q0, 448.0f, amax), kInv448, q0);
  t.s = s;
  t.slow = amax_bits != 0 && amax_bits < kMarksteinMinAmaxBits;
  t.xscale = t.slow ? 0x1p64f : 1.0f;
  const float div = s * t.xscale;
  const float y = __builtin_amdgcn_rcpf(div);
  const float r = __builtin_fmaf(__builtin_fmaf(-div, y, 1.0f), y, y);
  t.div = amax_bits ? div : 1.0f;
  t.mul = amax_bits ? r : 1.0f;
  t.neg_e = 0;
  return t;
}

__device__ __forceinline__ TileScale tile_scale_pow2(uint32_t amax_bits) {
  TileScale t;
  t.slow = false;
  t.div = 1.0f;
  t.mul = 1.0f;
  t.xscale = 1.0f;
  if (amax_bits == 0) {
    t.s = 0.0f;
    t.neg_e = 0;
    return t;
  }
  int ebits = (int)(amax_bits >> 7);
  int mant = (int)(amax_bits & 0x7F);
  int E;
  bool above;  // significand of amax > 1.75 (448 = 1.75 * 2^8)
  if (ebits != 0) {
    E = ebits - 127;
    above = mant > 0x60;
  } else {  // BF16 subnormal: amax = mant * 2^-133
    int p = 31 - __clz(mant);
    E = p - 133;
    above = (mant * 4) > (7 << p);
  }
  int e = E - 8 + (above ? 1 : 0);
  uint32_t sbits = e >= -126 ? (uint32_t)(e + 127) << 23 : 1u << (e + 149);
  t.s = __uint_as_float(sbits);
  t.neg_e = -e;
  return t;
}

__device__ __forceinline__ float quotient_free(float x, const TileScale& t) {
  const float xs = x * t.xscale;
  const float q0 = xs * t.mul;
  const float e = __builtin_fmaf(-q0, t.div, xs);
  return __builtin_copysignf(__builtin_fmaf(e, t.mul, q0), x);  // keeps -0 for negative zero inputs
}

template <bool POW2>
__device__ __forceinline__ float quotient(float x, const TileScale& t) {
  if constexpr (POW2) {
    return __builtin_ldexpf(x, t.neg_e);
  } else {
    return quotient_free(x, t);
  }
}

template <bool POW2>
__device__ __forceinline__ TileScale tile_scale(uint32_t amax_bits) {
  if constexpr (POW2) {
    return tile_scale_pow2(amax_bits);
  } else {
    return tile_scale_free(amax_bits);
  }
}

// Runs body(q) with q(x) = the tile quotient of x.  Free scales: the
// multiplication of x by 2^64 for a tiny-amax tile is taken only when some
// lane of the wave holds such a tile (a wave-uniform branch: call it with
// every lane of the wave active), so the common case is the bare Markstein
// quotient.
template <bool POW2, class Body>
__device__ __forceinline__ auto with_quotient(const TileScale& t, Body body) {
  if constexpr (POW2) {
    return body([&](float x) { return quotient<true>(x, t); });
  } else {
    if (__builtin_amdgcn_ballot_w64(t.slow) == 0) {
      return body([&](float x) {
        const float q0 = x * t.mul;
        const float e = __builtin_fmaf(-q0, t.div, x);
        return __builtin_copysignf(__builtin_fmaf(e, t.mul, q0), x);
      });
    }
    return body([&](float x) { return quotient_free(x, t); });
  }
}

// The sign bits of four BF16 values (words a, b: low half first) as the
// sign bits of four code bytes, in pack4_e4m3's order.
__device__ __forceinline__ uint32_t signs4(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07050301u) & 0x80808080u;
}

// Eight BF16 values (one 16-byte chunk) -> eight codes (two words), free
// scales.  The Markstein quotient goes without its copysign: it already
// carries the sign of every nonzero input, and OR-ing the inputs' sign bits
// into the codes restores the one it loses, that of -0 (+0 / s and -0 / s
// both come out +0).  SCALED: x is first multiplied by the tile's xscale
// (2^64 for a tiny-amax tile, else 1); without it the caller has checked
// that no tile of its wave is tiny.
template <bool SCALED>
__device__ __forceinline__ uint2 encode8_markstein(uint4 v, const TileScale& t) {
  auto q = [&](float x) {
    const float xs = SCALED ? x * t.xscale : x;
    const float q0 = xs * t.mul;
    const float e = __builtin_fmaf(-q0, t.div, xs);
    return __builtin_fmaf(e, t.mul, q0);
  };
  uint2 r;
  r.x = pack4_e4m3(q(bf16_lo(v.x)), q(bf16_hi(v.x)), q(bf16_lo(v.y)), q(bf16_hi(v.y))) | signs4(v.x, v.y);
  r.y = pack4_e4m3(q(bf16_lo(v.z)), q(bf16_hi(v.z)), q(bf16_lo(v.w)), q(bf16_hi(v.w))) | signs4(v.z, v.w);
  return r;
}

// Eight BF16 values -> eight codes.  Free scales: the multiplication by 2^64
// of a tiny-amax tile is taken only when some lane of the wave holds such a
// tile (a wave-uniform branch: call it with every lane of the wave active).
template <bool POW2>
__device__ __forceinline__ uint2 encode8(uint4 v, const TileScale& t) {
  if constexpr (POW2) {
    return with_quotient<true>(t, [&](auto q) {
      uint2 r;
      r.x = pack4_e4m3(q(bf16_lo(v.x)), q(bf16_hi(v.x)), q(bf16_lo(v.y)), q(bf16_hi(v.y)));
      r.y = pack4_e4m3(q(bf16_lo(v.z)), q(bf16_hi(v.z)), q(bf16_lo(v.w)), q(bf16_hi(v.w)));
      return r;
    });
  } else {
    if (__builtin_amdgcn_ballot_w64(t.slow) == 0) return encode8_markstein<false>(v, t);
    return encode8_markstein<true>(v, t);
  }
}

// Lane n of each 16-lane DPP row, broadcast to the row (row_newbcast).
template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + N, 0xF, 0xF, false);
}
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __uint_as_float(row_bcast<N>(__float_as_uint(v)));
}

// Loads up to 8 BF16 values (nvalid may be <= 0 or >= 8); missing ones are +0.
__device__ __forceinline__ uint4 load8_masked(const uint16_t* p, int nvalid) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (2 * i < nvalid) ? (uint32_t)p[2 * i] : 0u;
    uint32_t hi = (2 * i + 1 < nvalid) ? (uint32_t)p[2 * i + 1] : 0u;
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void store8_masked(uint8_t* p, uint2 c, int nvalid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < nvalid) p[i] = (uint8_t)(((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFF);
  }
}

}  // namespace fp8q
