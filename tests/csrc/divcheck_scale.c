/* Exhaustive host check of the quotient method used with a static scale:
 * for a normal finite scale s the device forms x / s as
 *     s' = |s| * 2^k in [1, 2);  r = 1 / s'   (once, IEEE division)
 *     x' = |x| * 2^k;  q0 = x' r;  e = fma(-q0, s', x');  q = fma(e, r, q0)
 * and must get the IEEE single-precision quotient bit for bit wherever the
 * E4M3 code depends on it.
 *
 * Reduction.  Every step commutes with scaling x' by a power of two 2^E as
 * long as q0, e and q stay normal (round to nearest is scale invariant and
 * the fma residual is exact).  The E4M3 code depends on the quotient only
 * for 2^-11 <= q < 2^10 (below, both round to the zero code; above, both
 * saturate to 448): there x' >= 2^-11 and every intermediate is far inside
 * the normal range.  So checking x' with exponent 0 is enough: x' = m_x in
 * [1, 2) runs over the 128 mantissas a bf16 input can have, s' over all
 * 2^23 fp32 mantissas in [1, 2): 2^30 pairs, each compared bit for bit with
 * x' / s'.  The two ends of the range that matters (x' exponents -11 and 9)
 * are run as well rather than taken from the scaling argument.
 * Prints "pairs mismatches" and exits 0 iff there are none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(void) {
  long long pairs = 0, bad = 0;
  static const int exps[3] = {0, -11, 9};
  for (int ei = 0; ei < 3; ++ei) {
    const uint32_t xexp = (uint32_t)(127 + exps[ei]) << 23;
#pragma omp parallel for reduction(+ : pairs, bad) schedule(dynamic, 4096)
  for (int32_t m = 0; m < (1 << 23); ++m) {
    const float sp = from_bits(0x3F800000u | (uint32_t)m);   /* [1, 2) */
    const float r = 1.0f / sp;
    for (uint32_t j = 0; j < 128; ++j) {
      const float xa = from_bits(xexp | (j << 16));           /* bf16 mantissa j */
      const float q0 = xa * r;
      const float er = fmaf(-q0, sp, xa);
      const float q = fmaf(er, r, q0);
      const float ref = xa / sp;
      ++pairs;
      if (to_bits(q) != to_bits(ref)) {
        ++bad;
        if (bad < 5) fprintf(stderr, "mismatch s'=%a x'=%a q=%a ref=%a\n", sp, xa, q, ref);
      }
    }
  }
  }
  printf("%lld %lld\n", pairs, bad);
  return bad != 0;
}
