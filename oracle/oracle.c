/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for counter-based bulk fills.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
 * CPU-baseline leg, never by the product path.  Shares no code with the HIP library.
 *
 * Every function is the plain definition written out one element at a time; no blocking,
 * no vectorisation, no reordering.  Built with -O2 -ffp-contract=off -fno-fast-math on
 * x86-64 SSE2, so every double and float operation is one IEEE-754 round-to-nearest-even
 * operation (perturbation-kernel, "Backends", §Why SIMD is exact: a fused multiply-add
 * rounds once where the reference rounds twice, so none is allowed here).
 *
 * Readings where the pages are silent are marked READING and listed in the design notes.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Substream positions a rejection loop may consume before it gives up.  Reaching it has
 * probability below 2^-65536 for every bound and layer; it only makes each function
 * total.  READING. */
#define SUBSTREAM_CAP 65536u

/* ---------------------------------------------------------------------------------
 * Generator layers.
 * Phobos stdlib, "Random numbers", §hash32: the lowbias32 hash in wrapping i32
 * arithmetic; its shifts are logical.  `_mix(x, s)` is read as x ^ (x >>> s), the
 * xorshift of lowbias32 (READING: _mix itself is not printed).
 * ------------------------------------------------------------------------------- */
static uint32_t mix(uint32_t x, unsigned s) { return x ^ (x >> s); }

uint32_t orc_hash32(uint32_t x)
{
    /* The page's constants are the i32 values 2146121005 and -2073254261; an i32
     * multiply that wraps is the u32 multiply of the same bits. */
    x = mix(x, 16);
    x = x * (uint32_t)2146121005;
    x = mix(x, 15);
    x = x * (uint32_t)-2073254261;
    x = mix(x, 16);
    return x;
}

/* Phobos, §uniform: the hash is taken of counter ^ hash32(seed). */
uint32_t orc_word(uint32_t key, uint32_t counter) { return orc_hash32(counter ^ orc_hash32(key)); }

/* Phobos, §uniform: low 23 bits times 2^-23 (the page writes 8388607 and
 * 1.1920928955078125e-7).  Both conversions are exact. */
float orc_uniform(uint32_t key, uint32_t counter)
{
    return (float)(orc_word(key, counter) & 8388607u) * 1.1920928955078125e-7f;
}

/* Phobos, §randn: Box-Muller of the uniforms at counters 2c and 2c+1, exactly as printed
 * (cos of 6.283185307179586 times the second uniform), evaluated in f64 and rounded once.
 * Used only as a special case the f32 normal fill must reduce to. */
float orc_randn(uint32_t key, uint32_t counter)
{
    double u1 = orc_uniform(key, 2u * counter);
    double u2 = orc_uniform(key, 2u * counter + 1u);
    return (float)(sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2));
}

/* tandem-sycl, "Design", §Normals: a miss continues on split(g) of sub(PURPOSE) of the
 * key, at position 0.  READING: sub(k, P) = hash32(hash32(k) ^ P), split(kP, g) =
 * word(kP, g), and the substream's word j is word(split, j). */
uint32_t orc_sub(uint32_t key, uint32_t purpose) { return orc_hash32(orc_hash32(key) ^ purpose); }
uint32_t orc_split(uint32_t key_p, uint32_t g) { return orc_word(key_p, g); }

static uint64_t draw64(uint32_t key, uint32_t i)
{
    /* READING: a 64-bit draw i is the word pair at counters 2i (low) and 2i+1 (high). */
    return (uint64_t)orc_word(key, 2u * i) | ((uint64_t)orc_word(key, 2u * i + 1u) << 32);
}

/* ---------------------------------------------------------------------------------
 * Draw sources.  Bounded draws, the ziggurat and Box-Muller are defined once over a
 * source: the lowbias32 stream of a 32-bit key, or Philox4x32-10 (defined further down)
 * of a 64-bit key.  A source gives word i, the 64-bit draw i (words 2i low, 2i+1 high)
 * and, for a purpose P, the substream of draw i:
 *   lowbias32: substream word j of draw i is word(split(sub(key, P), i), j) (above);
 *   Philox, READING: substream word j of draw i is lane j & 3 of the Philox block of the
 *     same key with counter (lo32 i, hi32 i, P, j >> 2).  The primary stream's blocks
 *     have counter words 2 and 3 zero, so P != 0 keeps the two disjoint.
 * A 64-bit substream draw j is substream words 2j (low) and 2j+1 (high).
 * ------------------------------------------------------------------------------- */
typedef struct {
    int philox;
    uint32_t key32;
    uint64_t key64;
} src_t;

static void philox_block(uint64_t key, const uint32_t ctr[4], uint32_t out[4]);

static src_t lowbias_src(uint32_t key)
{
    src_t s = {0, key, 0};
    return s;
}

static src_t philox_src(uint64_t key)
{
    src_t s = {1, 0, key};
    return s;
}

static uint32_t philox_ctr_word(uint64_t key, uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                uint32_t lane)
{
    uint32_t ctr[4] = {c0, c1, c2, c3}, out[4];
    philox_block(key, ctr, out);
    return out[lane];
}

static uint32_t src_word(const src_t *s, uint64_t i)
{
    if (!s->philox) return orc_word(s->key32, (uint32_t)i);
    uint64_t b = i >> 2;
    return philox_ctr_word(s->key64, (uint32_t)b, (uint32_t)(b >> 32), 0u, 0u, (uint32_t)(i & 3u));
}

static uint64_t src_draw64(const src_t *s, uint64_t i)
{
    return (uint64_t)src_word(s, 2u * i) | ((uint64_t)src_word(s, 2u * i + 1u) << 32);
}

static uint32_t src_sub_word(const src_t *s, uint32_t purpose, uint64_t i, uint32_t j)
{
    if (!s->philox) return orc_word(orc_split(orc_sub(s->key32, purpose), (uint32_t)i), j);
    return philox_ctr_word(s->key64, (uint32_t)i, (uint32_t)(i >> 32), purpose, j >> 2, j & 3u);
}

static uint64_t src_sub_draw64(const src_t *s, uint32_t purpose, uint64_t i, uint32_t j)
{
    return (uint64_t)src_sub_word(s, purpose, i, 2u * j) | ((uint64_t)src_sub_word(s, purpose, i, 2u * j + 1u) << 32);
}

/* ---------------------------------------------------------------------------------
 * Draw-index checks.  Counters are 32-bit (the Phobos hash takes an i32); a fill whose
 * draws would need a counter at or beyond 2^32 is refused rather than wrapped.
 * READING.
 * ------------------------------------------------------------------------------- */
#define MAX_DRAW_W32 0xFFFFFFFFull          /* one word per draw */
#define MAX_DRAW_W64 0x7FFFFFFFull          /* two words per draw */
#define MAX_DRAW_U16 0x1FFFFFFFFull         /* two draws per word */
#define MAX_DRAW_U8 0x3FFFFFFFFull          /* four draws per word */
#define MAX_DRAW_BOOL 0x1FFFFFFFFFull       /* 32 draws per word */

static int check_draws(uint64_t start, uint64_t n, const uint64_t *draws, uint64_t dmax)
{
    if (draws) {
        for (uint64_t k = 0; k < n; ++k)
            if (draws[k] > dmax) return ORC_ERANGE;
        return ORC_OK;
    }
    if (n == 0) return ORC_OK;
    if (start > dmax || n - 1 > dmax - start) return ORC_ERANGE;
    return ORC_OK;
}

#define DRAW(k) (draws ? draws[(k)] : start + (k))
#define CHECK(dmax)                                                      \
    do {                                                                 \
        if (n && !out) return ORC_EINVAL;                                \
        int rc_ = check_draws(start, n, draws, (dmax));                  \
        if (rc_) return rc_;                                             \
    } while (0)

/* ---------------------------------------------------------------------------------
 * Uniform fills.  tandem-cuda, "Performance", §GPU: narrow types write fewer bytes of
 * the same stream (READING: u16 draw i is half i&1 of word i>>1, u8 draw i is byte i&3
 * of word i>>2, little-endian); tandem-sycl, "Design", §Fills: a bool is one byte per
 * bit (READING: bool draw i is bit i&31 of word i>>5).
 * ------------------------------------------------------------------------------- */
int orc_fill_u32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint32_t *out)
{
    CHECK(MAX_DRAW_W32);
    for (uint64_t k = 0; k < n; ++k) out[k] = orc_word(key, (uint32_t)DRAW(k));
    return ORC_OK;
}

int orc_fill_u64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint64_t *out)
{
    CHECK(MAX_DRAW_W64);
    for (uint64_t k = 0; k < n; ++k) out[k] = draw64(key, (uint32_t)DRAW(k));
    return ORC_OK;
}

static uint16_t draw16(uint32_t key, uint64_t d)
{
    return (uint16_t)(orc_word(key, (uint32_t)(d >> 1)) >> (16u * (unsigned)(d & 1u)));
}

int orc_fill_u16(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint16_t *out)
{
    CHECK(MAX_DRAW_U16);
    for (uint64_t k = 0; k < n; ++k) out[k] = draw16(key, DRAW(k));
    return ORC_OK;
}

int orc_fill_u8(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint8_t *out)
{
    CHECK(MAX_DRAW_U8);
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t d = DRAW(k);
        out[k] = (uint8_t)(orc_word(key, (uint32_t)(d >> 2)) >> (8u * (unsigned)(d & 3u)));
    }
    return ORC_OK;
}

int orc_fill_bool(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint8_t *out)
{
    CHECK(MAX_DRAW_BOOL);
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t d = DRAW(k);
        out[k] = (uint8_t)((orc_word(key, (uint32_t)(d >> 5)) >> (unsigned)(d & 31u)) & 1u);
    }
    return ORC_OK;
}

/* f32: Phobos, §uniform, exactly. */
int orc_fill_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(MAX_DRAW_W32);
    for (uint64_t k = 0; k < n; ++k) out[k] = orc_uniform(key, (uint32_t)DRAW(k));
    return ORC_OK;
}

/* f64: READING: the low 53 bits of the 64-bit draw times 2^-53 (the f32 rule widened). */
int orc_fill_f64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, double *out)
{
    CHECK(MAX_DRAW_W64);
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t d = draw64(key, (uint32_t)DRAW(k));
        out[k] = (double)(d & ((1ull << 53) - 1u)) * 0x1p-53;
    }
    return ORC_OK;
}

/* f16 bits: READING: the binary16 encoding of (u16 draw & 0x7FF) * 2^-11, a uniform on a
 * 2^-11 grid in [0, 1).  The encoding is built field by field: for m in [2^e, 2^(e+1))
 * the value is 1.f * 2^(e-11), biased exponent e + 4, fraction m shifted to 10 bits. */
static uint16_t half_of_grid(uint32_t m)
{
    if (m == 0) return 0;
    int e = 0;
    while ((m >> (e + 1)) != 0) ++e;
    return (uint16_t)(((uint32_t)(e + 4) << 10) | ((m << (10 - e)) & 0x3FFu));
}

int orc_fill_f16_bits(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint16_t *out)
{
    CHECK(MAX_DRAW_U16);
    for (uint64_t k = 0; k < n; ++k) out[k] = half_of_grid(draw16(key, DRAW(k)) & 0x7FFu);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * Bounded integers.  perturbation-kernel, "Backends", §Why the GPU can be exact names
 * Lemire's multiply-shift with rejection; tandem-cuda, "Performance", §GPU: a rejection
 * is rare and its retry runs out of line.  READING: the exact threshold of Lemire (2019),
 * t = (2^W - s) mod s: reject while the low half of x*s is below t; a rejected draw
 * continues on split(g) of sub(key, BL32 or BL64), positions 0, 1, 2, ...
 * ------------------------------------------------------------------------------- */
/* One multiply-shift step: the value is the high half of x * s, and x is accepted iff
 * the low half is at least t. */
static int lemire32_step(uint32_t x, uint32_t s, uint32_t t, uint32_t *r)
{
    uint64_t m = (uint64_t)x * s;
    *r = (uint32_t)(m >> 32);
    return (uint32_t)m >= t;
}

static int lemire64_step(uint64_t x, uint64_t s, uint64_t t, uint64_t *r)
{
    unsigned __int128 m = (unsigned __int128)x * s;
    *r = (uint64_t)(m >> 64);
    return (uint64_t)m >= t;
}

static uint32_t lemire32_src(const src_t *src, uint64_t i, uint32_t s)
{
    uint32_t t = (uint32_t)(0u - s) % s, r;
    if (lemire32_step(src_word(src, i), s, t, &r)) return r;
    for (uint32_t j = 0; j < SUBSTREAM_CAP; ++j)
        if (lemire32_step(src_sub_word(src, ORC_P_BELOW32, i, j), s, t, &r)) break;
    return r;
}

static uint64_t lemire64_src(const src_t *src, uint64_t i, uint64_t s)
{
    uint64_t t = (0ull - s) % s, r;
    if (lemire64_step(src_draw64(src, i), s, t, &r)) return r;
    for (uint32_t j = 0; j < SUBSTREAM_CAP; ++j)
        if (lemire64_step(src_sub_draw64(src, ORC_P_BELOW64, i, j), s, t, &r)) break;
    return r;
}

uint32_t orc_lemire32(uint32_t key, uint32_t i, uint32_t s)
{
    src_t src = lowbias_src(key);
    return lemire32_src(&src, i, s);
}

uint64_t orc_lemire64(uint32_t key, uint32_t i, uint64_t s)
{
    src_t src = lowbias_src(key);
    return lemire64_src(&src, i, s);
}

/* The multiply-shift step alone over given words (no hashing, no retry), so a test can
 * sweep every 32-bit word. */
int orc_lemire32_map(const uint32_t *x, uint64_t n, uint32_t s, uint32_t *out, uint8_t *accepted)
{
    if (s == 0 || (n && (!x || !out || !accepted))) return ORC_EINVAL;
    uint32_t t = (uint32_t)(0u - s) % s;
    for (uint64_t k = 0; k < n; ++k) accepted[k] = (uint8_t)lemire32_step(x[k], s, t, &out[k]);
    return ORC_OK;
}

int orc_lemire64_map(const uint64_t *x, uint64_t n, uint64_t s, uint64_t *out, uint8_t *accepted)
{
    if (s == 0 || (n && (!x || !out || !accepted))) return ORC_EINVAL;
    uint64_t t = (0ull - s) % s;
    for (uint64_t k = 0; k < n; ++k) accepted[k] = (uint8_t)lemire64_step(x[k], s, t, &out[k]);
    return ORC_OK;
}

int orc_fill_u32_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       uint32_t bound, uint32_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    CHECK(MAX_DRAW_W32);
    for (uint64_t k = 0; k < n; ++k) out[k] = orc_lemire32(key, (uint32_t)DRAW(k), bound);
    return ORC_OK;
}

int orc_fill_u64_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       uint64_t bound, uint64_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    CHECK(MAX_DRAW_W64);
    for (uint64_t k = 0; k < n; ++k) out[k] = orc_lemire64(key, (uint32_t)DRAW(k), bound);
    return ORC_OK;
}

/* tandem-cuda, "Performance", §GPU table: *_below "with a low bound" into int32_t and
 * int64_t; the value is low + (bounded draw).  A range whose top exceeds the type is
 * refused. */
int orc_fill_i32_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       int32_t low, uint32_t bound, int32_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    if ((int64_t)low + (int64_t)bound - 1 > (int64_t)INT32_MAX) return ORC_ERANGE;
    CHECK(MAX_DRAW_W32);
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (int32_t)((int64_t)low + orc_lemire32(key, (uint32_t)DRAW(k), bound));
    return ORC_OK;
}

int orc_fill_i64_below32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                         int64_t low, uint32_t bound, int64_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    if ((__int128)low + (__int128)bound - 1 > (__int128)INT64_MAX) return ORC_ERANGE;
    CHECK(MAX_DRAW_W32);
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (int64_t)((__int128)low + orc_lemire32(key, (uint32_t)DRAW(k), bound));
    return ORC_OK;
}

int orc_fill_i64_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       int64_t low, uint64_t bound, int64_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    if ((__int128)low + (__int128)bound - 1 > (__int128)INT64_MAX) return ORC_ERANGE;
    CHECK(MAX_DRAW_W64);
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (int64_t)((__int128)low + orc_lemire64(key, (uint32_t)DRAW(k), bound));
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * f64 normal: the 1024-layer ziggurat.  tandem-sycl, "Design", §Normals: one 64-bit draw
 * per element, element i takes draw i, about 0.43 % of draws miss the fast path and
 * continue on split(i) of sub(key, PURPOSE_NORMAL64) at position 0.
 * The layer table is the Marsaglia-Tsang equal-area construction (ziggurat.c).
 * READING (layout of a draw d): layer L = d & 1023, sign = bit 10, u = (d >> 11) * 2^-53.
 * Fast path: x = u * X[L]; accept iff x < X[L+1].  Wedge (L >= 1): one substream draw e,
 * y = (e >> 11) * 2^-53, accept x iff F[L] + y * (F[L+1] - F[L]) < exp(-x*x/2), else the
 * next substream draw restarts as a primary draw.  Tail (L = 0): two substream draws a, b
 * give ua, ub in (0, 1]; xi = -ln(ua) / r, eta = -ln(ub); accept r + xi iff
 * 2 eta > xi^2, else draw the next pair.  The sign is that of the draw that missed.
 * ------------------------------------------------------------------------------- */
#define ZIG_LAYERS 1024u
static double zig_x[ZIG_LAYERS + 1], zig_f[ZIG_LAYERS + 1], zig_r;
static int zig_ready;

static void zig_init(void)
{
    if (zig_ready) return;
    double v;
    orc_zig_table(ZIG_LAYERS, zig_x, zig_f, &zig_r, &v);
    zig_ready = 1;
}

static double unit53(uint64_t d) { return (double)(d >> 11) * 0x1p-53; }

static double zig_normal(const src_t *src, uint64_t i, uint8_t *path)
{
    uint64_t d = src_draw64(src, i);
    uint32_t j = 0; /* next substream position (64-bit draws) */
    int restarted = 0;
    for (;;) {
        uint32_t L = (uint32_t)(d & (ZIG_LAYERS - 1u));
        int neg = (int)((d >> 10) & 1u);
        double x = unit53(d) * zig_x[L];
        if (x < zig_x[L + 1]) {
            if (path) *path = restarted ? 3 : 0;
            return neg ? -x : x;
        }
        if (L == 0) {
            for (;;) {
                if (j + 2 > SUBSTREAM_CAP) return NAN;
                uint64_t a = src_sub_draw64(src, ORC_P_NORMAL64, i, j++);
                uint64_t b = src_sub_draw64(src, ORC_P_NORMAL64, i, j++);
                double ua = (double)((a >> 11) + 1u) * 0x1p-53;
                double ub = (double)((b >> 11) + 1u) * 0x1p-53;
                double xi = -log(ua) / zig_r;
                double eta = -log(ub);
                if (eta + eta > xi * xi) {
                    if (path) *path = 2;
                    double t = zig_r + xi;
                    return neg ? -t : t;
                }
            }
        }
        if (j + 1 > SUBSTREAM_CAP) return NAN;
        double y = unit53(src_sub_draw64(src, ORC_P_NORMAL64, i, j++));
        double fy = zig_f[L] + y * (zig_f[L + 1] - zig_f[L]);
        if (fy < exp(-0.5 * (x * x))) {
            if (path) *path = 1;
            return neg ? -x : x;
        }
        if (j + 1 > SUBSTREAM_CAP) return NAN;
        d = src_sub_draw64(src, ORC_P_NORMAL64, i, j++);
        restarted = 1;
    }
}

int orc_fill_normal_f64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        double *out, uint8_t *path)
{
    CHECK(MAX_DRAW_W64);
    zig_init();
    src_t src = lowbias_src(key);
    for (uint64_t k = 0; k < n; ++k)
        out[k] = zig_normal(&src, DRAW(k), path ? path + k : NULL);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * f32 normal: Box-Muller pairs.  tandem-sycl, "Design", §Normals: float normals are
 * Box-Muller pairs with the angle moved into [-pi, pi); Phobos, §randn: the pair for
 * counter c is the uniforms at 2c and 2c+1, r = sqrt(-2 log(1 - u1)).
 * READING: draw i belongs to pair c = i >> 1; even i takes r cos(theta), odd i r sin(theta);
 * the angle is 2 pi t with t = u2 - 1 when u2 >= 1/2, else u2 (a whole turn, so cos(theta)
 * equals Phobos randn's cos(2 pi u2)).  Evaluated in f64 from the exact f32 uniforms and
 * rounded once to f32.
 * ------------------------------------------------------------------------------- */
static float unit23_of(uint32_t w) { return (float)(w & 8388607u) * 1.1920928955078125e-7f; }

static float box_muller(const src_t *src, uint64_t i, int half_turn)
{
    uint64_t c = i >> 1;
    float u1 = unit23_of(src_word(src, 2u * c));
    float u2 = unit23_of(src_word(src, 2u * c + 1u));
    double r = sqrt(-2.0 * log(1.0 - (double)u1));
    double t;
    if (half_turn) t = (double)u2 - 0.5;
    else t = u2 >= 0.5f ? (double)u2 - 1.0 : (double)u2;
    double theta = 6.283185307179586 * t;
    return (float)((i & 1u) ? r * sin(theta) : r * cos(theta));
}

int orc_fill_normal_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(MAX_DRAW_W32);
    src_t src = lowbias_src(key);
    for (uint64_t k = 0; k < n; ++k) out[k] = box_muller(&src, DRAW(k), 0);
    return ORC_OK;
}

/* tandem-sycl, "Design", §Normals: the float normal fill shifts the angle by half a turn
 * into [-pi, pi).  READING: t = u2 - 1/2, so theta = 2 pi u2 - pi and both values are the
 * negation of the whole-turn fill's (cos and sin of theta - pi); same pairs and radius. */
int orc_fill_normal_f32_half_turn(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(MAX_DRAW_W32);
    src_t src = lowbias_src(key);
    for (uint64_t k = 0; k < n; ++k) out[k] = box_muller(&src, DRAW(k), 1);
    return ORC_OK;
}

/* Phobos, §randn: one normal per counter, randn(key, c) for c = start + k, exactly as the
 * page prints it (orc_randn).  Counters c < 2^31 (words 2c and 2c+1). */
int orc_fill_randn_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(0x7FFFFFFFull);
    for (uint64_t k = 0; k < n; ++k) out[k] = orc_randn(key, (uint32_t)DRAW(k));
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * Exponentials.  tandem-sycl, "Design", §Exponentials and tandem-cuda, "Performance",
 * §GPU: the f32 exponential keeps every draw within 0.571 ulp so that 1 - exp(-x) maps
 * back to the draw's own 2^-24 grid point; the f64 one uses an f64 logarithm.
 * READING: x = -ln(1 - u) (inversion), +0.0 at u = 0.
 *   f64: u = the f64 uniform of the draw, (d & (2^53 - 1)) * 2^-53, x in f64.
 *   f32: u = (word & 0xFFFFFF) * 2^-24 (the low 24 bits), x = -ln(1 - u) rounded once to
 *        f32 (evaluated in f64; 1 - u is exact in both).
 * ------------------------------------------------------------------------------- */
static double neg_log1m(double u)
{
    double l = log(1.0 - u);
    return l == 0.0 ? 0.0 : -l;
}

int orc_fill_exponential_f64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, double *out)
{
    CHECK(MAX_DRAW_W64);
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t d = draw64(key, (uint32_t)DRAW(k));
        out[k] = neg_log1m((double)(d & ((1ull << 53) - 1u)) * 0x1p-53);
    }
    return ORC_OK;
}

int orc_fill_exponential_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(MAX_DRAW_W32);
    for (uint64_t k = 0; k < n; ++k) {
        uint32_t w = orc_word(key, (uint32_t)DRAW(k));
        out[k] = (float)neg_log1m((double)(w & 0xFFFFFFu) * 0x1p-24);
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * Dropout.  Phobos, §dropout: where(uniform(seed, counter) >= p, x / (1 - p), 0) with
 * p in [0, 1); the counter is the element's flat index.  1 - p and the quotient are f32
 * operations (a true division, not a multiply by a reciprocal).
 * ------------------------------------------------------------------------------- */
int orc_dropout_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float p,
                    const float *x, float *y, uint8_t *mask)
{
    if (!(p >= 0.0f && p < 1.0f)) return ORC_EINVAL;
    if (n && (!x || !y)) return ORC_EINVAL;
    int rc = check_draws(start, n, draws, MAX_DRAW_W32);
    if (rc) return rc;
    float q = 1.0f - p;
    for (uint64_t k = 0; k < n; ++k) {
        int keep = orc_uniform(key, (uint32_t)DRAW(k)) >= p;
        y[k] = keep ? x[k] / q : 0.0f;
        if (mask) mask[k] = (uint8_t)keep;
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * Weighted choice.  tandem-sycl, "Design", §Fills: the choice fill maps each 64-bit draw
 * through an alias table.  The table's construction is not on the pages; READING: Vose's
 * alias method in integers.  Each index j gets an integer mass m_j out of n * 2^32,
 * m_j = floor(w_j / S * n 2^32), the rounding remainder going to the largest weight
 * (lowest index on ties).  Columns hold 2^32 each: small = {m < 2^32}, large = the rest,
 * both FIFO in index order; a small s takes q[s] = m_s and alias[s] = front of large,
 * whose mass drops by 2^32 - m_s and moves it to the back of small once below 2^32.
 * Columns left over hold exactly 2^32: q = 0, alias = itself.
 * Map of draw d: column = (hi32(d) * n) >> 32, coin = lo32(d);
 * out = coin < q[column] ? column : alias[column].
 * ------------------------------------------------------------------------------- */
int orc_alias_build(const double *w, uint32_t n, uint32_t *q, uint32_t *alias, uint64_t *mass)
{
    if (!w || !q || !alias || n == 0 || n > (1u << 24)) return ORC_EINVAL;
    double s = 0.0;
    for (uint32_t j = 0; j < n; ++j) {
        if (!(w[j] >= 0.0) || !isfinite(w[j])) return ORC_EINVAL;
        s += w[j];
    }
    if (!(s > 0.0) || !isfinite(s)) return ORC_EINVAL;

    const uint64_t col = 1ull << 32;
    const uint64_t total = (uint64_t)n << 32;
    uint64_t *m = (uint64_t *)malloc(sizeof(uint64_t) * n);
    uint32_t *small = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *large = (uint32_t *)malloc(sizeof(uint32_t) * n);
    if (!m || !small || !large) {
        free(m); free(small); free(large);
        return ORC_EINVAL;
    }
    uint64_t sum = 0;
    uint32_t jmax = 0;
    for (uint32_t j = 0; j < n; ++j) {
        m[j] = (uint64_t)floor(w[j] / s * (double)total);
        sum += m[j];
        if (w[j] > w[jmax]) jmax = j;
    }
    m[jmax] = (uint64_t)((int64_t)m[jmax] + ((int64_t)total - (int64_t)sum));
    if (mass) memcpy(mass, m, sizeof(uint64_t) * n);

    uint32_t ns_head = 0, ns_tail = 0, nl_head = 0, nl_tail = 0;
    for (uint32_t j = 0; j < n; ++j) {
        if (m[j] < col) small[ns_tail++] = j;
        else large[nl_tail++] = j;
    }
    /* `small` can grow by at most n entries in total: each index enters it once. */
    while (ns_head < ns_tail && nl_head < nl_tail) {
        uint32_t sidx = small[ns_head++];
        uint32_t lidx = large[nl_head];
        q[sidx] = (uint32_t)m[sidx];
        alias[sidx] = lidx;
        m[lidx] -= col - m[sidx];
        if (m[lidx] < col) {
            ++nl_head;
            small[ns_tail++] = lidx;
        }
    }
    while (nl_head < nl_tail) {
        uint32_t j = large[nl_head++];
        q[j] = 0;
        alias[j] = j;
    }
    while (ns_head < ns_tail) { /* unreachable with exact integer masses */
        uint32_t j = small[ns_head++];
        q[j] = 0;
        alias[j] = j;
    }
    free(m); free(small); free(large);
    return ORC_OK;
}

int orc_fill_choice_u32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        const uint32_t *q, const uint32_t *alias, uint32_t ncat, uint32_t *out)
{
    if (ncat == 0 || !q || !alias) return ORC_EINVAL;
    CHECK(MAX_DRAW_W64);
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t d = draw64(key, (uint32_t)DRAW(k));
        uint32_t column = (uint32_t)(((d >> 32) * (uint64_t)ncat) >> 32);
        uint32_t coin = (uint32_t)d;
        out[k] = coin < q[column] ? column : alias[column];
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), the counter-based generator behind
 * the comparison column of tandem-cuda, "Performance".  Key (lo, hi); block b has counter
 * (lo32 b, hi32 b, 0, 0); word 4b + j is output lane j.  Each round multiplies lanes 0 and
 * 2 by 0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the next state is
 * (hi(lane2 product) ^ lane1 ^ k0, lo(lane2 product), hi(lane0 product) ^ lane3 ^ k1,
 * lo(lane0 product)); the key is bumped by 0x9E3779B9 and 0xBB67AE85 between rounds.
 * Pinned against rocRAND's Philox4x32-10 (an independent implementation): its words for
 * seed s, subsequence q and offset o equal these for key s and counter words 2-3 = q, from
 * word o (tests/test_oracle_philox_rocrand.py).
 * ------------------------------------------------------------------------------- */
static void philox_block(uint64_t key, const uint32_t ctr[4], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = (uint32_t)key, k1 = (uint32_t)(key >> 32);
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    for (int j = 0; j < 4; ++j) out[j] = c[j];
}

static uint32_t philox_word(uint64_t key, uint64_t w)
{
    uint64_t b = w >> 2;
    return philox_ctr_word(key, (uint32_t)b, (uint32_t)(b >> 32), 0u, 0u, (uint32_t)(w & 3u));
}

#define MAX_DRAW_PHILOX_W32 0xFFFFFFFFFFFFFFFFull
#define MAX_DRAW_PHILOX_W64 0x7FFFFFFFFFFFFFFFull

int orc_philox_fill_u32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint32_t *out)
{
    CHECK(MAX_DRAW_PHILOX_W32);
    for (uint64_t k = 0; k < n; ++k) out[k] = philox_word(key, DRAW(k));
    return ORC_OK;
}

static uint64_t philox_draw64(uint64_t key, uint64_t i)
{
    return (uint64_t)philox_word(key, 2u * i) | ((uint64_t)philox_word(key, 2u * i + 1u) << 32);
}

int orc_philox_fill_u64(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint64_t *out)
{
    CHECK(MAX_DRAW_PHILOX_W64);
    for (uint64_t k = 0; k < n; ++k) out[k] = philox_draw64(key, DRAW(k));
    return ORC_OK;
}

int orc_philox_fill_f32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(MAX_DRAW_PHILOX_W32);
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (float)(philox_word(key, DRAW(k)) & 8388607u) * 1.1920928955078125e-7f;
    return ORC_OK;
}

int orc_philox_fill_f64(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws, double *out)
{
    CHECK(MAX_DRAW_PHILOX_W64);
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (double)(philox_draw64(key, DRAW(k)) & ((1ull << 53) - 1u)) * 0x1p-53;
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------
 * Philox variants of the bounded, choice and normal fills: the same definitions as the
 * lowbias32 fills above over the Philox source (src_t): word i, 64-bit draw i, and the
 * per-draw substreams with counter (lo32 i, hi32 i, P, j >> 2).  The word source, primary
 * and substream counters alike, is pinned against rocRAND's engine.
 * ------------------------------------------------------------------------------- */
/* Substream word j of draw i for purpose P (exposed for the tests). */
uint32_t orc_philox_sub_word(uint64_t key, uint64_t i, uint32_t purpose, uint32_t j)
{
    src_t src = philox_src(key);
    return src_sub_word(&src, purpose, i, j);
}

int orc_philox_fill_u32_below(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                              uint32_t bound, uint32_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    CHECK(MAX_DRAW_PHILOX_W32);
    src_t src = philox_src(key);
    for (uint64_t k = 0; k < n; ++k) out[k] = lemire32_src(&src, DRAW(k), bound);
    return ORC_OK;
}

int orc_philox_fill_u64_below(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                              uint64_t bound, uint64_t *out)
{
    if (bound == 0) return ORC_EINVAL;
    CHECK(MAX_DRAW_PHILOX_W64);
    src_t src = philox_src(key);
    for (uint64_t k = 0; k < n; ++k) out[k] = lemire64_src(&src, DRAW(k), bound);
    return ORC_OK;
}

int orc_philox_fill_choice_u32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                               const uint32_t *q, const uint32_t *alias, uint32_t ncat, uint32_t *out)
{
    if (ncat == 0 || !q || !alias) return ORC_EINVAL;
    CHECK(MAX_DRAW_PHILOX_W64);
    src_t src = philox_src(key);
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t d = src_draw64(&src, DRAW(k));
        uint32_t column = (uint32_t)(((d >> 32) * (uint64_t)ncat) >> 32);
        uint32_t coin = (uint32_t)d;
        out[k] = coin < q[column] ? column : alias[column];
    }
    return ORC_OK;
}

int orc_philox_fill_normal_f32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out)
{
    CHECK(MAX_DRAW_PHILOX_W32);
    src_t src = philox_src(key);
    for (uint64_t k = 0; k < n; ++k) out[k] = box_muller(&src, DRAW(k), 0);
    return ORC_OK;
}

int orc_philox_fill_normal_f64(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                               double *out, uint8_t *path)
{
    CHECK(MAX_DRAW_PHILOX_W64);
    zig_init();
    src_t src = philox_src(key);
    for (uint64_t k = 0; k < n; ++k) out[k] = zig_normal(&src, DRAW(k), path ? path + k : NULL);
    return ORC_OK;
}
