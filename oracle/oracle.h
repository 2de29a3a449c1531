/*
 * oracle.h -- plain, slow, single-threaded CPU oracle for counter-based bulk fills.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link, load or
 * call this code: only the test suite, the package's smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source with the HIP library and reads nothing
 * the HIP library produces.
 *
 * Every function writes out[k] = T(key, d_k) for k < n, where d_k = start + k, or
 * d_k = draws[k] when `draws` is not NULL (a gather at arbitrary draw indices, used
 * for sampled comparisons at full size).  Return: 0 ok, 1 bad argument, 2 a draw
 * index outside the counter space.
 *
 * Sources (pages named by title and section):
 *   Phobos stdlib, "Random numbers": §hash32, §uniform, §randn, §dropout, and the
 *     figure "Counter-based random numbers on a tile".
 *   tandem-sycl, "Design": §Fills (element i takes draw i, bool = one byte per bit,
 *     choice through an alias table), §Normals (1024-layer ziggurat, misses continue on
 *     split(g) of sub(PURPOSE_NORMAL64) at position 0; Box-Muller pairs for floats).
 *   tandem-cuda, "Performance": §GPU table (row names fix the fill family: u8, u16,
 *     f16 bits, u32, u64, f32, f64, bool, *_below with and without a low bound).
 *   perturbation-kernel, "Backends", §Why the GPU can be exact (Lemire multiply-shift
 *     with rejection).
 * Methods the pages name but do not define follow the published papers: Marsaglia &
 * Tsang (2000) for the ziggurat construction, Lemire (2019) for the exact rejection
 * threshold, Vose (1991) for the alias table, Salmon et al. (SC'11) for Philox4x32-10.
 *
 * orc_philox_*: the Philox4x32-10 word source is pinned against rocRAND's implementation
 * (primary and substream counters, offsets past 2^34 words); the Philox bounded, choice
 * and normal variants reduce to pinned maps over it.
 */
#ifndef BULK_FILLS_ORACLE_H
#define BULK_FILLS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_ERANGE = 2 };

/* Purpose tags for sub(key, P): ASCII "NORM", "BL32", "BL64". */
#define ORC_P_NORMAL64 0x4E4F524Du
#define ORC_P_BELOW32 0x424C3332u
#define ORC_P_BELOW64 0x424C3634u

/* Generator layers, exposed so each can be pinned separately. */
uint32_t orc_hash32(uint32_t x);
uint32_t orc_word(uint32_t key, uint32_t counter);       /* hash32(counter ^ hash32(key)) */
float orc_uniform(uint32_t key, uint32_t counter);       /* low 23 bits times 2^-23 */
float orc_randn(uint32_t key, uint32_t counter);         /* Phobos randn, evaluated in f64 */
uint32_t orc_sub(uint32_t key, uint32_t purpose);        /* hash32(hash32(key) ^ purpose) */
uint32_t orc_split(uint32_t key_p, uint32_t g);          /* word(key_p, g) */
uint32_t orc_lemire32(uint32_t key, uint32_t i, uint32_t s);
uint64_t orc_lemire64(uint32_t key, uint32_t i, uint64_t s);
int orc_lemire32_map(const uint32_t *x, uint64_t n, uint32_t s, uint32_t *out, uint8_t *accepted);
int orc_lemire64_map(const uint64_t *x, uint64_t n, uint64_t s, uint64_t *out, uint8_t *accepted);

/* Uniform fills. */
int orc_fill_u8(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint8_t *out);
int orc_fill_u16(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint16_t *out);
int orc_fill_u32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint32_t *out);
int orc_fill_u64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint64_t *out);
int orc_fill_f16_bits(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint16_t *out);
int orc_fill_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float *out);
int orc_fill_f64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, double *out);
int orc_fill_bool(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, uint8_t *out);

/* Bounded fills: values in [0, bound) or [low, low + bound). */
int orc_fill_u32_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       uint32_t bound, uint32_t *out);
int orc_fill_u64_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       uint64_t bound, uint64_t *out);
int orc_fill_i32_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       int32_t low, uint32_t bound, int32_t *out);
int orc_fill_i64_below32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                         int64_t low, uint32_t bound, int64_t *out);
int orc_fill_i64_below(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       int64_t low, uint64_t bound, int64_t *out);

/* Normals.  `path` (nullable) receives 0 = fast path, 1 = wedge, 2 = tail, 3 = a
 * restart ended in the fast path; used by the tests to count misses. */
int orc_fill_normal_f64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        double *out, uint8_t *path);
int orc_fill_normal_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        float *out);
/* The pages' half-turn Box-Muller (angle 2 pi u2 - pi): the negation of the above. */
int orc_fill_normal_f32_half_turn(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                                  float *out);
/* Phobos randn, one normal per counter: element k = randn(key, start + k). */
int orc_fill_randn_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                       float *out);

/* Exponentials: x = -ln(1 - u); f64 from the f64 uniform, f32 from a 2^-24 grid (rounded
 * once from f64). */
int orc_fill_exponential_f64(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                             double *out);
int orc_fill_exponential_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                             float *out);

/* Dropout: y[k] = u >= p ? x[k] / (1 - p) : 0, u the uniform at draw d_k. */
int orc_dropout_f32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws, float p,
                    const float *x, float *y, uint8_t *mask);

/* Alias table (integer Vose build) and the choice fill through it. */
int orc_alias_build(const double *weights, uint32_t n, uint32_t *q, uint32_t *alias,
                    uint64_t *mass);
int orc_fill_choice_u32(uint32_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        const uint32_t *q, const uint32_t *alias, uint32_t ncat,
                        uint32_t *out);

/* Ziggurat layer table for `nlayers` layers, built in binary128 and rounded once:
 * x[0..nlayers], f[0..nlayers], r, v.  x must hold nlayers+1 values, f likewise. */
int orc_zig_table(uint32_t nlayers, double *x, double *f, double *r, double *v);

/* Philox4x32-10 word source (64-bit key, block counter = word index / 4). */
int orc_philox_fill_u32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        uint32_t *out);
int orc_philox_fill_u64(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        uint64_t *out);
int orc_philox_fill_f32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        float *out);
int orc_philox_fill_f64(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                        double *out);

/* Philox variants of the bounded, choice and normal fills (same definitions over the
 * Philox source; a rejected or missed draw i continues on Philox blocks with counter
 * (lo32 i, hi32 i, purpose, j >> 2)). */
uint32_t orc_philox_sub_word(uint64_t key, uint64_t i, uint32_t purpose, uint32_t j);
int orc_philox_fill_u32_below(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                              uint32_t bound, uint32_t *out);
int orc_philox_fill_u64_below(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                              uint64_t bound, uint64_t *out);
int orc_philox_fill_choice_u32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                               const uint32_t *q, const uint32_t *alias, uint32_t ncat, uint32_t *out);
int orc_philox_fill_normal_f32(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                               float *out);
int orc_philox_fill_normal_f64(uint64_t key, uint64_t start, uint64_t n, const uint64_t *draws,
                               double *out, uint8_t *path);

#ifdef __cplusplus
}
#endif
#endif
