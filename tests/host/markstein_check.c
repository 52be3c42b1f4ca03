/* Exhaustive host check of the quantizers' element quotient.
 *
 * The 1x128 / 128x128 quantizers form a tile's scale s = RN32(amax / 448)
 * and r = RN32(1 / s) (without divisions; scale_reciprocal_check.c shows both
 * equal the IEEE results), and each element's quotient RN32(x / s) -- the
 * value the E4M3 rounding then reads -- with one Markstein correction of the
 * product by the rounded reciprocal (M. Markstein, "Computation of
 * elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
 * Dev. 34(1), 1990):
 *   r = RN32(1 / s), q0 = RN32(x * r), e = fma(-q0, s, x), q = fma(e, r, q0).
 * For every BF16 amax >= 2^-90 (exponent field >= 37) and every BF16 x with
 * |x| <= amax this program checks that q equals the IEEE quotient x / s, or
 * that both are at most 2^-10 in magnitude (then both encode to the E4M3
 * zero of x's sign).  Each step is odd in x, so x >= 0 covers the negatives.
 *
 * Tiles with 0 < amax < 2^-90 scale both operands by 2^64 first (exact: x
 * and s are at least 2^-149, and x * 2^64, s * 2^64 are normal):
 *   s' = s * 2^64, r' = RN32(1 / s'), x' = x * 2^64, then the same three
 * steps on (x', s', r').  x' / s' = x / s, and the second loop checks that
 * sequence against the IEEE quotient x / s for every such amax (including
 * those whose s is subnormal) and every BF16 x with |x| <= amax.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off markstein_check.c -o markstein_check
 * (fmaf must be a single rounding: the hardware instruction with -mfma, or
 * glibc's correctly rounded fmaf).  Prints the counts and returns 0 when
 * every pair agrees.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t bits) {
  uint32_t u = bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  const float tiny = 0x1p-10f;
  uint64_t pairs = 0, equal = 0, both_zero = 0, bad = 0;
  for (uint32_t ab = 37u << 7; ab <= 0x7F7Fu; ++ab) {
    const float amax = bf16(ab);
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      const float x = bf16(xb);
      const float ieee = x / s;
      const float q0 = x * r;
      const float e = fmaf(-q0, s, x);
      const float q = fmaf(e, r, q0);
      ++pairs;
      if (q == ieee) {
        ++equal;
      } else if (fabsf(q) <= tiny && fabsf(ieee) <= tiny) {
        ++both_zero;
      } else {
        if (bad < 10)
          printf("mismatch: amax bits 0x%04x x bits 0x%04x: markstein %a ieee %a\n", ab, xb, q, ieee);
        ++bad;
      }
    }
  }
  printf("pairs %llu equal %llu both-below-2^-10 %llu mismatches %llu\n", (unsigned long long)pairs,
         (unsigned long long)equal, (unsigned long long)both_zero, (unsigned long long)bad);

  /* tiny tiles: both operands scaled by 2^64 */
  uint64_t tpairs = 0, tequal = 0, tboth = 0, tbad = 0;
  const float k = 0x1p64f;
  for (uint32_t ab = 1; ab < (37u << 7); ++ab) {
    const float amax = bf16(ab);
    const float s = amax / 448.0f;
    const float s2 = s * k;
    const float r2 = 1.0f / s2;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      const float x = bf16(xb);
      const float ieee = x / s;
      const float x2 = x * k;
      const float q0 = x2 * r2;
      const float e = fmaf(-q0, s2, x2);
      const float q = fmaf(e, r2, q0);
      ++tpairs;
      if (q == ieee) {
        ++tequal;
      } else if (fabsf(q) <= tiny && fabsf(ieee) <= tiny) {
        ++tboth;
      } else {
        if (tbad < 10)
          printf("tiny mismatch: amax bits 0x%04x x bits 0x%04x: scaled markstein %a ieee %a\n", ab, xb, q, ieee);
        ++tbad;
      }
    }
  }
  printf("tiny pairs %llu equal %llu both-below-2^-10 %llu mismatches %llu\n", (unsigned long long)tpairs,
         (unsigned long long)tequal, (unsigned long long)tboth, (unsigned long long)tbad);
  return bad == 0 && tbad == 0 ? 0 : 1;
}
