/*
 * tk_device_api.h -- per-element draws for use inside HIP kernels (gfx950, wave64).
 *
 * Phobos stdlib, "Random numbers": a value is a hash of a seed and the element's own
 * counter, so it can be computed in registers inside the statement that uses it, and the
 * same (seed, counter) gives the same value on every call -- which is how a backward pass
 * redraws its forward pass's dropout mask instead of storing it.
 *
 * Every function here is the element function of a libtk fill (include/tk.h), and the
 * fill kernels are built from these same definitions, so for the same key
 *     tk_uniform_f32(hk, c)      == element c of tk_fill_f32(key, 0, ...)
 *     tk_uniform_f64(hk, i)      == element i of tk_fill_f64(key, 0, ...)
 *     tk_randn2_f32(hk, c, ...)  == elements 2c, 2c+1 of tk_fill_normal_f32(key, 0, ...)
 *     tk_dropout_apply_f32(x, p, q, hk, c) == y[c] of tk_dropout_f32(key, 0, ..., x, y, ...)
 * bit for bit, where hk = tk_key_hash(key) (computed once, on the host or the device).
 * Counters are 32-bit: a kernel that needs more than 2^32 words per key takes a new key.
 *
 * Counters (Phobos, §Random numbers): a counter must be unique across the whole launch,
 * which a block-local index is not; the element's global flat index is.  tk_randn*_f32
 * consumes two words per counter (2c and 2c+1), so mixed uses of one key need disjoint
 * counter ranges, or different keys.
 *
 * Each float transform is a fixed sequence of IEEE operations and gfx950 hardware
 * instructions with nothing a compiler may contract, so the values do not depend on the
 * caller's floating-point flags.
 */
#ifndef TK_DEVICE_API_H
#define TK_DEVICE_API_H

#include <hip/hip_runtime.h>
#include <stdint.h>

/* lowbias32 (Phobos, §hash32): three logical xorshifts and two wrapping multiplies by the
 * page's i32 constants 2146121005 and -2073254261, taken as u32 bit patterns. */
__host__ __device__ __forceinline__ uint32_t tk_hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

/* The per-key constant of every draw: hash32(key). */
__host__ __device__ __forceinline__ uint32_t tk_key_hash(uint32_t key) { return tk_hash32(key); }

/* Word c of the stream of key (Phobos, §uniform: hash32(counter ^ hash32(seed))). */
__device__ __forceinline__ uint32_t tk_word(uint32_t hk, uint32_t c) { return tk_hash32(c ^ hk); }

/* (w & 0x7FFFFF) * 2^-23, built as the float 1.m minus 1 (exact). */
__device__ __forceinline__ float tk_unit23(uint32_t w) {
  return __uint_as_float((w & 0x7FFFFFu) | 0x3F800000u) - 1.0f;
}

/* Uniform on the 2^-23 grid of [0, 1) (Phobos, §uniform). */
__device__ __forceinline__ float tk_uniform_f32(uint32_t hk, uint32_t c) { return tk_unit23(tk_word(hk, c)); }

/* Uniform on the 2^-53 grid of [0, 1): the low 53 bits of the 64-bit draw i, whose words
 * are 2i (low) and 2i+1 (high).  i < 2^31. */
__device__ __forceinline__ double tk_uniform_f64(uint32_t hk, uint32_t i) {
  const uint32_t lo = tk_word(hk, 2u * i), hi = tk_word(hk, 2u * i + 1u);
  return (double)(hi & 0x1FFFFFu) * 0x1p-21 + (double)lo * 0x1p-53;
}

/* Box-Muller of the f32 uniforms of words w1 and w2 (Phobos, §randn; the pair's second
 * value is r sin): r = sqrt(-2 ln(1 - u1)) from the hardware base-2 logarithm and square
 * root, the angle 2 pi t with t = u2 wrapped into [-1/2, 1/2) through the hardware sine
 * and cosine, which take turns.  Within 1.2e-6 of the exact pair; |x| < 5.65.
 * Both inputs come from the float 1.m of the word's low 23 bits m, each in one exact
 * subtraction: 1 - u1 = 2 - 1.m, and t = f - 3/2 where f is 1.m with bit 22 of m
 * flipped, which is 3/2 + u2 for u2 < 1/2 and 1/2 + u2 otherwise. */
__device__ __forceinline__ void tk_box_muller_f32(uint32_t w1, uint32_t w2, float *cos_part, float *sin_part) {
  const float one_minus_u1 = 2.0f - __uint_as_float((w1 & 0x7FFFFFu) | 0x3F800000u);
  const float t = __uint_as_float((w2 & 0x7FFFFFu) ^ 0x3FC00000u) - 1.5f;
  const float r = __builtin_amdgcn_sqrtf(__builtin_amdgcn_logf(one_minus_u1) * -1.38629436111989061883f);
  *cos_part = r * __builtin_amdgcn_cosf(t);
  *sin_part = r * __builtin_amdgcn_sinf(t);
}

/* The same pair with the angle shifted by half a turn (tandem-sycl, "Design", §Normals):
 * t = u2 - 1/2 (= 1.m - 3/2, exact), so both values are the negation of
 * tk_box_muller_f32's. */
__device__ __forceinline__ void tk_box_muller_half_turn_f32(uint32_t w1, uint32_t w2, float *cos_part,
                                                            float *sin_part) {
  const float one_minus_u1 = 2.0f - __uint_as_float((w1 & 0x7FFFFFu) | 0x3F800000u);
  const float t = __uint_as_float((w2 & 0x7FFFFFu) | 0x3F800000u) - 1.5f;
  const float r = __builtin_amdgcn_sqrtf(__builtin_amdgcn_logf(one_minus_u1) * -1.38629436111989061883f);
  *cos_part = r * __builtin_amdgcn_cosf(t);
  *sin_part = r * __builtin_amdgcn_sinf(t);
}

/* Box-Muller pair c of key hk: the words 2c and 2c+1.  c < 2^31. */
__device__ __forceinline__ void tk_randn2_f32(uint32_t hk, uint32_t c, float *cos_part, float *sin_part) {
  tk_box_muller_f32(tk_word(hk, 2u * c), tk_word(hk, 2u * c + 1u), cos_part, sin_part);
}

/* One standard normal per counter (Phobos, §randn: the cosine of pair c). */
__device__ __forceinline__ float tk_randn_f32(uint32_t hk, uint32_t c) {
  float a, b;
  tk_randn2_f32(hk, c, &a, &b);
  return a;
}

/* Whether dropout keeps element c: its uniform is at least p (Phobos, §dropout). */
__device__ __forceinline__ bool tk_dropout_keep(float p, uint32_t hk, uint32_t c) {
  return tk_uniform_f32(hk, c) >= p;
}

/* Dropout of x at counter c (Phobos, §dropout): x / (1 - p) if kept, else +0.0.  q is the
 * f32 value 1.0f - p, computed once by the caller; the quotient is the IEEE division.
 * Applied to the output gradient it is also the backward pass (same p, key, counters). */
__device__ __forceinline__ float tk_dropout_apply_f32(float x, float p, float q, uint32_t hk, uint32_t c) {
  return tk_dropout_keep(p, hk, c) ? __fdiv_rn(x, q) : 0.0f;
}

#endif /* TK_DEVICE_API_H */
