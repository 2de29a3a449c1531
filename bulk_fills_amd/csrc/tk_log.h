// tk_log.h -- the logarithms of the exponential fills: -ln x for x = 1 - u in (0, 1].
//
// Both reduce after Tang (1990, ACM TOMS 16(4)) with a short multiplier per table entry,
// so that the reduced argument is exact after one fused multiply-add:
//     x = 2^-n z' (z' in [0.6875, 1.375)),  -ln x = n ln 2 + ln v_j - ln(1 + q),
//     q = z' v_j - 1,
// where z' is z in [1, 2) (the mantissa) or, from the entry that starts at 1.375 on, z / 2,
// and the kernels compute q as z m_j - 1 with the halving folded into the stored m_j.  The
// tables and their derivation are in gen_log_table.py (log256.inc for f64, logf256.inc for
// f32).  The fills read them from an LDS copy per work-group: as L1 gathers the reads kept
// the texture addresser ~95 % busy (rocprofv3 TA_TA_BUSY) and bounded the fills.  The f64
// fill widens each entry to three whole doubles in its copy (LogEntryWide), so that an
// element's read needs no register moves to rebuild a double from its high word: ~1.5 %
// faster than reading the 16-byte entry, with the same values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "log256.inc"
#include "logf256.inc"

namespace tk {

// f64: one 16-byte entry per 1/256 of the mantissa range.
struct LogEntryD {
  double l_hi;       // ln v_j, a multiple of 2^-45
  uint32_t m_hi;     // high word of the multiplier m_j (9 significant bits: low word zero)
  uint32_t l_lo_hi;  // high word of ln v_j - l_hi (21 significant bits: low word zero)
};
static_assert(sizeof(LogEntryD) == 16, "one 16-byte load per entry in the LDS copy");

// The LDS form of an entry: the same three values, each a whole double.
struct LogEntryWide {
  double l_hi, m, l_lo;
};

__device__ __forceinline__ double log_m(const LogEntryD &t) { return __hiloint2double((int)t.m_hi, 0); }
__device__ __forceinline__ double log_m(const LogEntryWide &t) { return t.m; }
__device__ __forceinline__ double log_l_lo(const LogEntryD &t) { return __hiloint2double((int)t.l_lo_hi, 0); }
__device__ __forceinline__ double log_l_lo(const LogEntryWide &t) { return t.l_lo; }

static __constant__ LogEntryD kLogTableD[TK_LOGD_ENTRIES] = {TK_LOGD_TABLE_ROWS};

static_assert(TK_LOGD_ENTRIES == 256 && TK_LOGD_SPLIT == 96, "index bits and the halving threshold below");

// -ln(1 - u) for the f64 exponential, u = (hi & (2^21 - 1)) 2^-21 + lo 2^-53 (the draw's low
// 53 bits); exactly +0 at u = 0.
//  - x 2^21 = B - lo 2^-32 with B = 2^21 - (hi & (2^21 - 1)) in [1, 2^21]: one fused
//    multiply-add of two exact conversions, exact (x 2^53 is an integer of at most 53 bits);
//  - n = 21 - e (20 - e for the halved entries, e the exponent of x 2^21, 0 <= n <= 53) in
//    one subtraction: the borrow out of the 20 fraction bits of the high word is the halving
//    test (fraction bits >= 0x60000), as in the f32 logarithm below;
//  - q = z m_j - 1 is exact: m_j has at most 9 significant bits and |q| < 2^-8, so the
//    exact value fits in 53 bits;
//  - ln(1 + q) - q = q^2 s(q), s the Taylor polynomial through q^5 (ln(1 + q) through q^7;
//    the next term is below 2^-59 of the result); w = n LN2_HI + l_hi is exact, w - q is
//    carried exactly as rh + rl (Fast2Sum: |w| >= |q| whenever w != 0), and the low parts
//    go in last.
// A CPU model of these operations (tests) finds at most 0.502 ulp of error over every point
// of the 2^-24 grid and 2^25 more points of the 2^-53 grid, and exact reductions throughout.
// 21 f64 operations (the frexp that gives z / 2 included) and no integer work for z, where
// the general Tang reduction (z - c_j, a product by 1 / c_j and its residual) with the
// conversion of u took 27.
template <class Entry>
__device__ __forceinline__ double neg_ln_draw53(uint32_t lo, uint32_t hi, const Entry *tab) {
  const uint32_t b = 0x200000u - (hi & 0x1FFFFFu);
  const double xs = __builtin_fma((double)lo, -0x1p-32, (double)b);  // x 2^21, exact
  const uint32_t xh = (uint32_t)__double2hiint(xs);
  const uint32_t j = (xh >> 12) & 0xFFu;
  const int32_t n = (int32_t)((((1044u << 20) | 0x5FFFFu) - xh) >> 20);
  // z / 2 in [0.5, 1) in one v_frexp_mant, and h = q / 2 = (z / 2) m - 1/2, exact as q is.
  // Every step below is the step on q with exact power-of-two scalings folded into its
  // constants (each value is 2^k times the one computed on q, and rounding commutes with the
  // scaling), so the result is bit for bit that of
  //     s = -1/2 + q/3 - q^2/4 + q^3/5 - q^4/6 + q^5/7 (Horner),  p = q^2 s,
  //     rh + rl = w - q (Fast2Sum),  -ln x = rh + (((n LN2_LO + l_lo) - p) + rl).
  const double zhalf = __builtin_amdgcn_frexp_mant(xs);
  const Entry t = tab[j];
  const double m = log_m(t);
  const double l_lo = log_l_lo(t);
  const double h = __builtin_fma(zhalf, m, -0.5);  // exact
  double s = __builtin_fma(32 * (1.0 / 7), h, -16 * (1.0 / 6));  // 16 s1
  s = __builtin_fma(s, h, 8 * (1.0 / 5));                        // 8 s2
  s = __builtin_fma(s, h, 4 * -0.25);                            // 4 s3
  s = __builtin_fma(s, h, 2 * (1.0 / 3));                        // 2 s4
  s = __builtin_fma(s, h, -0.5);                                 // s
  const double p4 = (h * h) * s;                                 // p / 4
  const double dn = (double)n;
  const double w = __builtin_fma(dn, TK_LN2_HI, t.l_hi);  // exact
  const double rh = __builtin_fma(h, -2.0, w);            // w - q rounded
  const double rl = __builtin_fma(h, -2.0, w - rh);       // (w - rh) - q, exact
  const double tail = __builtin_fma(p4, -4.0, __builtin_fma(dn, TK_LN2_LO, l_lo)) + rl;
  return rh + tail;
}

// -ln(k 2^-24) rounded to f32 for the f32 exponential, k = 2^24 - m, 0 <= m < 2^24 (x = 1 - u
// with u = m 2^-24, exact).  Its own table (logf256.inc): k as a double is exact and carries
// the reduction directly (k = 2^e z, z in [1, 2)), the 8 leading fraction bits pick entry j,
// and from entry 96 on z is halved into [0.6875, 1) as in Tang's method.  The entry's
// multiplier v_j has at most 24 significant bits, so q = z v_j - 1 is exact in one fused
// multiply-add (z has at most 24 significant bits as well); the table stores v_j / 2 for
// the halved entries, so z itself never changes.  Then
//     -ln x = n ln 2 + ln v_j - ln(1 + q),   ln(1 + q) = q (1 - q/2 + q^2/3 - q^3/4),
// |q| <= 2^-9 (2^-8 at j = 0), n = 24 - e (23 - e for the halved entries), evaluated as
// fma(-q, u, w) with u the degree-3 factor and w = n ln 2 + ln v_j: ten f64 operations
// (with the conversions and the frexp that takes z / 2 from k), where the f64 logarithm
// above takes twenty.  n comes from one subtraction: the
// borrow out of the 20 fraction bits of k's high word is exactly the halving test (fraction
// bits >= 0x60000).  A CPU model of exactly these operations over all 2^24 inputs (tests)
// gives the correctly rounded f32 at every one, the worst error being 0.28 of the distance
// from the exact value to the nearest f32 rounding boundary.  +0 at m = 0.
struct LogEntryF {
  double m, l;  // multiplier of z in [1, 2) (v_j, or v_j / 2 from entry TK_LOGF_SPLIT on), ln v_j
};

static __constant__ LogEntryF kLogTableF[TK_LOGF_ENTRIES] = {TK_LOGF_TABLE_ROWS};

constexpr double kLn2 = 0x1.62e42fefa39efp-1;  // ln 2 rounded to nearest

static_assert(TK_LOGF_ENTRIES == 256 && TK_LOGF_SPLIT == 96, "index bits and the halving threshold below");

__device__ __forceinline__ float neg_ln_grid24_f32(uint32_t m, const LogEntryF *tab) {
  const uint32_t k = 0x1000000u - m;
  const double xk = (double)k;  // exact: k <= 2^24
  const uint32_t xh = (uint32_t)__double2hiint(xk);
  const uint32_t j = (xh >> 12) & 0xFFu;
  // 1047 - (xh >> 20), less one when the fraction bits reach 0x60000 (entry 96): 0 <= n <= 24
  const int32_t n = (int32_t)((0x4175FFFFu - xh) >> 20);
  // z / 2 = k 2^-(e+1) in [0.5, 1) in one v_frexp_mant, and h = q / 2 = (z / 2) m - 1/2,
  // exact as q is.  The polynomial runs on h with its coefficients scaled by powers of two
  // (8 s, then 4 (s q - 1/2), then 2 u), which gives bit for bit the values of
  //     s = 1/3 - q/4,  u = 1 + q (s q - 1/2),  -ln x = w - q u
  // evaluated on q (every step is the same rounding of an exactly scaled value).
  const double zhalf = __builtin_amdgcn_frexp_mant(xk);
  const LogEntryF t = tab[j];
  const double h = __builtin_fma(zhalf, t.m, -0.5);  // exact
  const double s8 = __builtin_fma(-4.0, h, 8.0 / 3);
  const double t2 = __builtin_fma(s8, h, -2.0);
  const double u2 = __builtin_fma(t2, h, 2.0);
  const double w = __builtin_fma((double)n, kLn2, t.l);
  return (float)__builtin_fma(-h, u2, w);
}

}  // namespace tk
