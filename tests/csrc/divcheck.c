/* Exhaustive host check of the quotient method used by the device
 * quantizers: for every positive finite bf16 amax and every bf16 x with
 * 0 <= x <= amax, the scaled reciprocal-plus-one-correction quotient
 *     s = amax / 448;  s' = s * 2^k in [1, 2);  r = 1 / s'
 *     x' = x * 2^k;  q0 = x' r;  e = fma(-q0, s', x');  q = fma(e, r, q0)
 * must equal the IEEE single-precision quotient x / s bit for bit, except
 * where both are <= 2^-10: every such value (half the smallest E4M3
 * subnormal, or less) encodes to the zero code of its sign, so the E4M3
 * code is the same.  Those exceptions come from x' falling into the fp32
 * subnormal range, where the residual e is not exact.
 * (Negative x give the negated result: every step is sign-symmetric.)
 * Prints "pairs bit_mismatches code_relevant_mismatches" and exits 0 iff
 * the last count is zero. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(void) {
  long long pairs = 0, diff = 0, bad = 0;
  const float zero_limit = 0x1p-10f;
#pragma omp parallel for reduction(+ : pairs, diff, bad) schedule(dynamic, 64)
  for (int ab = 1; ab < 0x7F80; ++ab) {
    float amax = from_bits((uint32_t)ab << 16);
    float s = amax / 448.0f;
    int e;
    (void)frexpf(s, &e);
    int k = 1 - e;
    float sp = ldexpf(s, k);
    float r = 1.0f / sp;
    for (int xb = 0; xb <= ab; ++xb) {
      float x = from_bits((uint32_t)xb << 16);
      float xa = ldexpf(x, k);
      float q0 = xa * r;
      float er = fmaf(-q0, sp, xa);
      float q = fmaf(er, r, q0);
      float ref = x / s;
      ++pairs;
      if (to_bits(q) != to_bits(ref)) {
        ++diff;
        if (!(q <= zero_limit && ref <= zero_limit)) {
          ++bad;
          if (bad < 5) fprintf(stderr, "mismatch amax=%a x=%a q=%a ref=%a\n", amax, x, q, ref);
        }
      }
    }
  }
  printf("%lld %lld %lld\n", pairs, diff, bad);
  return bad != 0;
}
