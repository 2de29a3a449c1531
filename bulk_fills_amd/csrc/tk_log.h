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
#include "logf256.inc"

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

// -ln(k 2^-24) rounded to f32 for the f32 exponential, k = 2^24 - m, 0 <= m < 2^24 (x = 1 - u
// with u = m 2^-24, exact).  Its own table (logf256.inc): k as a double is exact and carries
// the reduction directly (k = 2^e z, z in [1, 2)), the 8 leading fraction bits pick entry j,
// and from entry 96 on z is halved into [0.6875, 1) as in Tang's method.  The entry's
// multiplier v_j has at most 24 significant bits, so q = z v_j - 1 is exact in one fused
// multiply-add (z has at most 24 significant bits as well); the table stores v_j / 2 for
// the halved entries, so z itself never changes.  Then
//     -ln x = n ln 2 + ln v_j - ln(1 + q),   ln(1 + q) = q (1 - q/2 + q^2/3 - q^3/4),
// |q| <= 2^-9 (2^-8 at j = 0), n = 24 - e (23 - e for the halved entries), evaluated as
// fma(-q, u, w) with u the degree-3 factor and w = n ln 2 + ln v_j: nine f64 operations,
// where the general logarithm above takes about 25.  n comes from one subtraction: the
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
  // z = k 2^-e in [1, 2): k's fraction bits under the exponent of 1, as one v_bitop3
  // (truth table 0xEA = (a & b) | c)
  const uint32_t zh = __builtin_amdgcn_bitop3_b32(xh, 0x000FFFFFu, 0x3FF00000u, 0xEA);
  const double z = __hiloint2double((int)zh, __double2loint(xk));
  const LogEntryF t = tab[j];
  const double q = __builtin_fma(z, t.m, -1.0);  // exact
  double s = __builtin_fma(-0.25, q, 1.0 / 3);
  s = __builtin_fma(s, q, -0.5);
  const double u = __builtin_fma(s, q, 1.0);
  const double w = __builtin_fma((double)n, kLn2, t.l);
  return (float)__builtin_fma(-q, u, w);
}

}  // namespace tk
