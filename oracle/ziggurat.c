/*
 * ziggurat.c -- the ziggurat layer table for the oracle, built in IEEE binary128.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * tandem-sycl, "Design", §Normals names a 1024-layer ziggurat whose construction lives in
 * an appendix that is not on the pages.  READING: the equal-area construction of
 * Marsaglia & Tsang (2000) over f(x) = exp(-x^2/2):
 *   v = r f(r) + integral_r^inf f = r f(r) + sqrt(pi/2) erfc(r / sqrt 2),
 *   X[1] = r, X[i+1] = f^-1(v / X[i] + f(X[i])) for i = 1 .. N-2,
 *   r chosen so that the top layer closes: X[N-1] (1 - f(X[N-1])) = v,
 *   X[0] = v / f(r) (the base strip, which holds the tail), X[N] = 0,
 *   F[i] = f(X[i]) for 1 <= i < N, F[N] = 1, F[0] = 0 (the strip's floor; never read).
 * Every layer i >= 1 is the rectangle [0, X[i]] x [F[i], F[i+1]] of area v.
 * r is found by bisection; everything is computed in binary128 and rounded once to
 * binary64 (a double recurrence loses up to thousands of ulps over 1024 layers).
 */
#include "oracle.h"

#include <quadmath.h>
#include <stdlib.h>

typedef __float128 quad;

static quad zf(quad x) { return expq(-x * x / 2); }
static quad zf_inv(quad y) { return sqrtq(-2 * logq(y)); }
static quad ztail(quad r) { return sqrtq(M_PIq / 2) * erfcq(r / M_SQRT2q); }
static quad zarea(quad r) { return r * zf(r) + ztail(r); }

/* Runs the recurrence for a trial r.  Returns -1 when r is too small (the layers reach
 * the top of the curve before the last one), +1 when r is too large (the top layer is
 * wider than v). */
static int zig_side(uint32_t N, quad r, quad *X)
{
    quad v = zarea(r);
    X[1] = r;
    for (uint32_t i = 1; i + 2 <= N; ++i) {
        quad y = v / X[i] + zf(X[i]);
        if (y >= 1) return -1;
        X[i + 1] = zf_inv(y);
    }
    quad top = X[N - 1] * (1 - zf(X[N - 1]));
    return top > v ? +1 : -1;
}

int orc_zig_table(uint32_t N, double *x, double *f, double *r_out, double *v_out)
{
    if (N < 4 || N > 65536 || !x || !f) return ORC_EINVAL;
    quad *X = (quad *)malloc(sizeof(quad) * (N + 1));
    if (!X) return ORC_EINVAL;
    quad lo = 1, hi = 10;
    for (int it = 0; it < 128; ++it) {
        quad mid = (lo + hi) / 2;
        if (zig_side(N, mid, X) < 0) lo = mid;
        else hi = mid;
    }
    quad r = (lo + hi) / 2;
    zig_side(N, r, X);
    quad v = zarea(r);
    X[0] = v / zf(r);
    X[N] = 0;
    for (uint32_t i = 0; i <= N; ++i) x[i] = (double)X[i];
    f[0] = 0.0;
    for (uint32_t i = 1; i < N; ++i) f[i] = (double)zf(X[i]);
    f[N] = 1.0;
    if (r_out) *r_out = (double)r;
    if (v_out) *v_out = (double)v;
    free(X);
    return ORC_OK;
}
