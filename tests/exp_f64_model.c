/* Host model of the f64 exponential's logarithm (bulk_fills_amd/csrc/tk_log.h,
 * neg_ln_draw53): the same operations in the same order on the same table (log256.inc),
 * in IEEE double with fused multiply-adds where the kernel fuses.  Inputs: every point of
 * the 2^-24 grid (u = i 2^-24), then 2^25 points of the 2^-53 grid from a xorshift
 * generator, a third of them pushed next to u = 0 or u = 1 (small m, or m near 2^53).  The
 * draw's high word carries random bits above the 21 the fill uses.  Each result is compared
 * with -ln(1 - u) in long double (64-bit significand: the reference is good to ~2^-63
 * relative).  Also checks that the reduction q = z m - 1 is exact (long double holds z m
 * exactly: 53 + 9 bits) and that u = 0 gives +0.
 * Prints: worst error in ulps of the result, inexact reductions, wrong zeros.
 * Built with gcc -O2 -ffp-contract=off (no contraction beyond the explicit fma calls). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "log256.inc"

struct Entry {
  double l_hi;
  uint32_t m_hi, l_lo_hi;
};
static const struct Entry kTab[TK_LOGD_ENTRIES] = {TK_LOGD_TABLE_ROWS};

static long inexact = 0;

static double from_words(uint32_t h, uint32_t l) {
  const uint64_t b = ((uint64_t)h << 32) | l;
  double d;
  memcpy(&d, &b, 8);
  return d;
}

static double model(uint32_t lo, uint32_t hi) {
  const uint32_t b = 0x200000u - (hi & 0x1FFFFFu);
  const double xs = fma((double)lo, -0x1p-32, (double)b);
  uint64_t bits;
  memcpy(&bits, &xs, 8);
  const uint32_t xh = (uint32_t)(bits >> 32), xl = (uint32_t)bits;
  const uint32_t j = (xh >> 12) & 0xFFu;
  const int32_t n = (int32_t)((((1044u << 20) | 0x5FFFFu) - xh) >> 20);
  (void)xl;
  int e;
  const double zhalf = frexp(xs, &e); /* the kernel's v_frexp_mant: z / 2 in [0.5, 1) */
  const double m = from_words(kTab[j].m_hi, 0), l_lo = from_words(kTab[j].l_lo_hi, 0);
  const double h = fma(zhalf, m, -0.5);
  if ((long double)h != (long double)zhalf * (long double)m - 0.5L) ++inexact;
  double s = fma(32 * (1.0 / 7), h, -16 * (1.0 / 6));
  s = fma(s, h, 8 * (1.0 / 5));
  s = fma(s, h, 4 * -0.25);
  s = fma(s, h, 2 * (1.0 / 3));
  s = fma(s, h, -0.5);
  const double p4 = (h * h) * s;
  const double dn = (double)n;
  const double w = fma(dn, TK_LN2_HI, kTab[j].l_hi);
  const double rh = fma(h, -2.0, w);
  const double rl = fma(h, -2.0, w - rh);
  const double tail = fma(p4, -4.0, fma(dn, TK_LN2_LO, l_lo)) + rl;
  return rh + tail;
}

#ifdef TK_MODEL_LIB
/* Library form (tests/build_exp_model.py): the model of each 64-bit draw d, whose low 53
 * bits are u 2^53, for the GPU test that the fill computes exactly these operations. */
void tk_model_neg_ln_batch(const uint64_t *d, double *out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = model((uint32_t)d[i], (uint32_t)(d[i] >> 32));
}
#else
static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}

int main(void) {
  const uint64_t mask53 = (1ull << 53) - 1;
  double worst = 0.0;
  long wrong_zero = 0;
  for (long i = 0; i < (1L << 24) + (1L << 25); ++i) {
    uint64_t mm;
    if (i < (1L << 24)) {
      mm = (uint64_t)i << 29;
    } else {
      mm = next() & mask53;
      const long r = i % 3;
      if (r == 1) mm &= (1ull << (next() % 54)) - 1;                    /* u near 0 */
      if (r == 2) mm = mask53 - (mm & ((1ull << (next() % 54)) - 1));    /* u near 1 */
    }
    const uint32_t lo = (uint32_t)mm, hi = (uint32_t)(mm >> 32) | ((uint32_t)next() & 0xFFE00000u);
    const double got = model(lo, hi);
    if (mm == 0) {
      if (!(got == 0.0 && !signbit(got))) ++wrong_zero;
      continue;
    }
    const long double r = -logl((long double)((1ull << 53) - mm) * 0x1p-53L);
    const double rd = (double)r;
    const double ulp = nextafter(rd, INFINITY) - rd;
    const double e = (double)(fabsl((long double)got - r) / ulp);
    if (e > worst) worst = e;
  }
  printf("%.6f %ld %ld\n", worst, inexact, wrong_zero);
  return 0;
}
#endif
