/* Host model of the f32 exponential's logarithm (bulk_fills_amd/csrc/tk_log.h,
 * neg_ln_grid24_f32): the same operations in the same order on the same table
 * (logf256.inc), in IEEE double with fused multiply-adds where the kernel fuses, over
 * every input m in [0, 2^24).  Each result is compared with the correctly rounded f32 of
 * -ln(1 - m 2^-24) obtained from long double (64-bit significand); an input whose exact
 * value lies too close to an f32 rounding boundary for long double to decide is counted
 * separately.  Prints: wrong, undecided, and the worst error of the unrounded model value
 * as a fraction of the distance from the exact value to the nearest rounding boundary.
 * Built with gcc -O2 -ffp-contract=off (no contraction beyond the explicit fma calls). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "logf256.inc"

static const double kTab[TK_LOGF_ENTRIES][2] = {TK_LOGF_TABLE_ROWS};
static const double kLn2 = 0x1.62e42fefa39efp-1;

static double model(uint32_t m) {
  const uint32_t k = 0x1000000u - m;
  const double xk = (double)k;
  uint64_t b;
  memcpy(&b, &xk, 8);
  const uint32_t xh = (uint32_t)(b >> 32), xl = (uint32_t)b;
  const uint32_t j = (xh >> 12) & 0xFFu;
  const int32_t n = (int32_t)((0x4175FFFFu - xh) >> 20);
  (void)xl;
  int e;
  const double zhalf = frexp(xk, &e); /* the kernel's v_frexp_mant: z / 2 in [0.5, 1) */
  const double h = fma(zhalf, kTab[j][0], -0.5);
  const double s8 = fma(-4.0, h, 8.0 / 3);
  const double t2 = fma(s8, h, -2.0);
  const double u2 = fma(t2, h, 2.0);
  const double w = fma((double)n, kLn2, kTab[j][1]);
  return fma(-h, u2, w);
}

int main(void) {
  long wrong = 0, undecided = 0;
  double worst = 0.0;
  for (uint32_t m = 0; m < (1u << 24); ++m) {
    const double d = model(m);
    const float got = (float)d;
    if (m == 0) {
      if (!(d == 0.0 && !signbit(d))) ++wrong;
      continue;
    }
    const long double r = -logl((long double)(0x1000000u - m) * 0x1p-24L);
    const float want = (float)r;
    const float nb = nextafterf(want, r > (long double)want ? INFINITY : 0.0f);
    const long double mid = ((long double)want + (long double)nb) / 2;
    const long double dist = fabsl(r - mid);
    if (dist < fabsl(r) * 0x1p-60L) {
      ++undecided;
      continue;
    }
    if (memcmp(&got, &want, 4) != 0) ++wrong;
    const long double e = fabsl((long double)d - r) / dist;
    if (e > worst) worst = (double)e;
  }
  printf("%ld %ld %.6f\n", wrong, undecided, worst);
  return 0;
}
