// tk_log.h -- -ln x for x in (0, 1], the logarithm of the exponential fills.
//
// Table-driven after Tang (1990, ACM TOMS 16(4)); the table and its derivation are in
// log128.inc and gen_log_table.py.  For x = 2^E z with z in [0.6875, 1.375):
//     -ln x = -E ln 2 - ln c_j - ln(1 + q),   q = (z - c_j) / c_j,  |q| <= 2^-8 (2^-7 at j = 0)
// q is carried as qh + ql (z - c_j is exact, and so is its residual after the product by
// 1/c_j), ln(1 + q) - q is its Taylor polynomial through q^7 (the next term is below
// 2^-59 of the result), -E ln 2 - ln c_j is split so that its high part is exact, and the
// high sum is made exact with Fast2Sum (|w| >= |qh| whenever w != 0).  Over all 2^24
// points of the 2^-24 grid and 2^26 random points of the 2^-53 grid the error is at most
// 0.514 ulp, and rounding it to f32 gives the correctly rounded f32 at every grid point.
// About 30 VALU operations and two 16-byte table reads; the compiler's log takes ~115.
// The fills read the table from an LDS copy per work-group: as L1 gathers the reads kept
// the texture addresser ~95 % busy (rocprofv3 TA_TA_BUSY) and bounded both fills.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "log128.inc"

namespace tk {

struct LogEntry {
  double invc, nlog_hi, nlog_lo, c;  // 1 / c_j, -ln c_j = nlog_hi + nlog_lo, c_j
};

static __constant__ LogEntry kLogTable[TK_LOG_ENTRIES] = {TK_LOG_TABLE_ROWS};

// -ln x for x in [2^-53, 1] (every 1 - u of the fills); exactly +0 at x = 1.  `tab` is
// kLogTable or a work-group's LDS copy of it.
__device__ __forceinline__ double neg_ln_unit(double x, const LogEntry *tab) {
  const uint32_t xh = (uint32_t)__double2hiint(x);
  const uint32_t j = (xh >> 13) & (TK_LOG_ENTRIES - 1);  // 7 leading fraction bits
  const bool half = j >= TK_LOG_SPLIT;
  const int32_t n = 1023 - (int32_t)(xh >> 20) - (half ? 1 : 0);  // -E, 0 <= n <= 53
  const uint32_t zh = (xh & 0x000FFFFFu) | (half ? 0x3FE00000u : 0x3FF00000u);
  const double z = __hiloint2double((int)zh, __double2loint(x));
  const LogEntry t = tab[j];
  const double f = z - t.c;                                   // exact
  const double qh = f * t.invc;
  const double ql = __builtin_fma(-qh, t.c, f) * t.invc;      // the residual is exact
  double s = __builtin_fma(1.0 / 7, qh, -1.0 / 6);            // ln(1+q) - q = q^2 s(q)
  s = __builtin_fma(s, qh, 1.0 / 5);
  s = __builtin_fma(s, qh, -0.25);
  s = __builtin_fma(s, qh, 1.0 / 3);
  s = __builtin_fma(s, qh, -0.5);
  const double p = (qh * qh) * s;
  const double dn = (double)n;
  const double w = __builtin_fma(dn, TK_LN2_HI, t.nlog_hi);   // exact
  const double rh = w - qh;
  const double rl = (w - rh) - qh;                            // exact
  const double tail = ((__builtin_fma(dn, TK_LN2_LO, t.nlog_lo) - ql) - p) + rl;
  return rh + tail;
}

// -ln x rounded to f32 for the f32 exponential's inputs x = 1 - m 2^-24, 0 <= m < 2^24.
// The same reduction as neg_ln_unit, but a degree-5 polynomial, no residual of q, no split
// of the constants and no compensated sum: about 13 f64 operations instead of ~25.  Its
// error is at most 6 % of the distance from the exact value to the nearest f32 rounding
// boundary at every one of the 2^24 inputs (a CPU model of these operations against long
// double over all of them; degree 4 would round 15 of them wrongly), so the result is the
// correctly rounded f32, as neg_ln_unit's rounded once.  +0 at x = 1.
__device__ __forceinline__ float neg_ln_grid24_f32(double x, const LogEntry *tab) {
  const uint32_t xh = (uint32_t)__double2hiint(x);
  const uint32_t j = (xh >> 13) & (TK_LOG_ENTRIES - 1);
  const bool half = j >= TK_LOG_SPLIT;
  const int32_t n = 1023 - (int32_t)(xh >> 20) - (half ? 1 : 0);
  const uint32_t zh = (xh & 0x000FFFFFu) | (half ? 0x3FE00000u : 0x3FF00000u);
  const double z = __hiloint2double((int)zh, __double2loint(x));
  const LogEntry t = tab[j];
  const double q = (z - t.c) * t.invc;
  double s = __builtin_fma(1.0 / 5, q, -0.25);
  s = __builtin_fma(s, q, 1.0 / 3);
  s = __builtin_fma(s, q, -0.5);
  const double p = (q * q) * s;
  const double w = __builtin_fma((double)n, TK_LN2_HI + TK_LN2_LO, t.nlog_hi + t.nlog_lo);
  return (float)((w - q) - p);
}

}  // namespace tk
