/* Exhaustive check of the quantizers' FP32 division (CPU, test only).
 *
 * The 1x128 quantizers compute q = enc(fl32(x / s)) with s = fl32(amax / 448)
 * (page 1 of the surveyed pages, the uniondaocoop.com post: one scale per
 * 1x128 activation tile, from the tile's maximum magnitude).  The kernels do
 * not divide per element: once per tile they take r = RN(1 / s') and then
 * evaluate, per element,
 *     p = x' * r;  t = fma(p, s', -x');  y = fma(-t, r, p)
 * (one Markstein correction of the product x' * r), where x' = x * sx and
 * s' = s * sx with sx = 2^64 for tiles whose amax is below 2^-60 and 1 else.
 * With power-of-two scales the kernels use y = x' * r alone (r is exact).
 *
 * This program replays exactly those float operations on the host (IEEE
 * binary32, round to nearest even, fused multiply-add) for every pair of
 * BF16 values (x, amax) with amax positive and finite and |x| <= amax, both
 * signs of x, with and without rounding the scale up to a power of two, and
 * compares y with the correctly rounded quotient w = fl32(x / s):
 *   - y must have the same bits as w, or
 *   - y and w must have the same sign and magnitudes at most 2^-10: both
 *     then encode to the E4M3 zero of that sign (the smallest E4M3 magnitude
 *     is 2^-9; half of it rounds to the even neighbour, zero).
 * The second case is where the correction step's preconditions fail: the
 * residual x' - p*s' (about 2^-24 |x'|) underflows when |x'| < 2^-102, or
 * the quotient itself is subnormal.  On the unscaled path s >= 2^-60 / 448,
 * so such an x gives |x / s| < 2^-33.
 * So every pair gives the E4M3 code of the correctly rounded quotient.
 * Prints the counts and exits 0 when every pair passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* next power of two at or above a positive finite float, on the bits */
static float pow2_up(float s) {
  uint32_t b = u_of(s);
  if (b >= 0x00800000u) {
    if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;
  } else if (b & (b - 1u)) {
    uint32_t p = 1u;
    while (p < b) p <<= 1;
    b = p;
  }
  return f_of(b);
}

int main(void) {
  volatile float k448 = 448.0f;
  long long pairs = 0, normal_eq = 0, sub_zero = 0, fails = 0;
  for (int pow2 = 0; pow2 < 2; ++pow2) {
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, normal_eq, sub_zero, fails)
    for (uint32_t ab = 1; ab < 0x7F80u; ++ab) {          /* positive finite BF16 amax */
      const float amax = f_of(ab << 16);
      float s = amax / k448;
      if (s < 0x1p-149f) s = 0x1p-149f;
      if (pow2) s = pow2_up(s);
      const float sx = amax < 0x1p-60f ? 0x1p64f : 1.0f;
      const float ss = s * sx;
      const float r = 1.0f / ss;
      for (uint32_t xb = 0; xb <= ab; ++xb) {
        for (int neg = 0; neg < 2; ++neg) {
          const float x = f_of((xb << 16) | (neg ? 0x80000000u : 0u));
          const float xs = x * sx;                         /* exact: a power of two */
          float y;
          if (pow2) {
            y = xs * r;
          } else {
            const float p = xs * r;
            const float t = fmaf(p, ss, -xs);
            y = fmaf(-t, r, p);
#ifdef PLANT_NO_CORRECTION   /* a planted mistake the check must catch */
            y = p;
#endif
          }
          const float want = x / s;                        /* IEEE: correctly rounded */
          ++pairs;
          if (u_of(y) == u_of(want)) {
            ++normal_eq;
          } else if ((u_of(y) >> 31) == (u_of(want) >> 31) && fabsf(y) <= 0x1p-10f && fabsf(want) <= 0x1p-10f) {
            ++sub_zero;
          } else {
            ++fails;
          }
        }
      }
    }
  }
  printf("pairs %lld bit-equal %lld both-encode-to-zero %lld failures %lld\n", pairs, normal_eq, sub_zero, fails);
  return fails == 0 && pairs > 0 ? 0 : 1;
}
