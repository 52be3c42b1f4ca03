/* Exhaustive host check of the quantizers' tile scale and its reciprocal.
 *
 * A free-scale tile has s = RN32(amax / 448) (the oracle's IEEE division) and
 * its element quotients use RN32(1 / div), div = s (or s * 2^64 for a tile
 * with 0 < amax < 2^-90).  The GPU forms neither with an IEEE division:
 *   s: q0 = RN32(amax * RN32(1/448)), e = fma(-q0, 448, amax),
 *      s = fma(e, RN32(1/448), q0)   (Markstein's correction, M. Markstein,
 *      IBM J. Res. Dev. 34(1), 1990);
 *   r: from the hardware reciprocal y (documented within 1 ulp of 1/div),
 *      one Newton step r = fma(fma(-div, y, 1), y, y).
 * For every nonzero finite BF16 amax this program checks that s equals
 * amax / 448 bit for bit (subnormal results included), and that r equals
 * 1.0f / div for every y within 2 ulps of it.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off scale_reciprocal_check.c -lm
 * (fmaf must round once: the hardware instruction with -mfma, or glibc's
 * correctly rounded fmaf).  Prints the counts; returns 0 when all agree.
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

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(void) {
  const float inv448 = 1.0f / 448.0f;
  long amaxes = 0, bad_s = 0, recips = 0, bad_r = 0;
  for (uint32_t ab = 1; ab <= 0x7F7Fu; ++ab) { /* every positive finite BF16 */
    const float amax = bf16(ab);
    const float ieee = amax / 448.0f;
    const float q0 = amax * inv448;
    const float s = fmaf(fmaf(-q0, 448.0f, amax), inv448, q0);
    ++amaxes;
    if (bits_of(s) != bits_of(ieee)) {
      if (bad_s < 10) printf("scale mismatch: amax %a: %a, IEEE %a\n", amax, s, ieee);
      ++bad_s;
    }
    const float div = ab < (37u << 7) ? ieee * 0x1p64f : ieee; /* 37 << 7: the BF16 pattern of 2^-90 */
    const float want = 1.0f / div;
    float y[5];
    y[0] = want;
    y[1] = nextafterf(want, 0.0f);
    y[2] = nextafterf(y[1], 0.0f);
    y[3] = nextafterf(want, INFINITY);
    y[4] = nextafterf(y[3], INFINITY);
    for (int i = 0; i < 5; ++i) {
      const float r = fmaf(fmaf(-div, y[i], 1.0f), y[i], y[i]);
      ++recips;
      if (bits_of(r) != bits_of(want)) {
        if (bad_r < 10) printf("reciprocal mismatch: div %a from %a: %a, IEEE %a\n", div, y[i], r, want);
        ++bad_r;
      }
    }
  }
  printf("amax values %ld scale mismatches %ld reciprocal starts %ld mismatches %ld\n", amaxes, bad_s, recips, bad_r);
  return (bad_s || bad_r) ? 1 : 0;
}
