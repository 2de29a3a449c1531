// tk_device.h -- device-side generator and transforms for gfx950 (wave64).
//
// Everything here is inline __device__ code used by the fill kernels.  Integer work is
// exact; floating-point transforms are either exact (uniform grids, the ziggurat fast
// path) or evaluated as single IEEE operations with contraction disabled at build time
// (-ffp-contract=off), so results match a plain CPU evaluation bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tk_device_api.h"

namespace tk {

constexpr int kBlock = 256;  // work-group size: four wave64s

// s_waitcnt immediate that waits for every outstanding vector memory operation of the wave
// (gfx9 encoding: vmcnt 0, expcnt and lgkmcnt at their maxima, i.e. not waited for)
constexpr unsigned kWaitVmcnt0 = 0x0F70u;

// ---- generator and f32 uniform: the public per-element API (include/tk_device_api.h),
// so that the fills and kernels written against that header draw the same values ------
__device__ __forceinline__ uint32_t lowbias32(uint32_t x) { return tk_hash32(x); }

// Word c of the stream keyed by hk = lowbias32(key) (Phobos, §uniform: counter ^ hash(seed)).
__device__ __forceinline__ uint32_t word(uint32_t hk, uint32_t c) { return tk_word(hk, c); }

// ---- exact uniform transforms ---------------------------------------------------------
// f32: (w & 0x7FFFFF) * 2^-23 (exact).
__device__ __forceinline__ float unit23(uint32_t w) { return tk_unit23(w); }

// f64: (d & (2^53-1)) * 2^-53 from the two words: hi's low 21 bits scaled by 2^-21 plus
// lo scaled by 2^-53.  Both terms and their sum are exact.
__device__ __forceinline__ double unit53_lowbits(uint32_t lo, uint32_t hi) {
  return (double)(hi & 0x1FFFFFu) * 0x1p-21 + (double)lo * 0x1p-53;
}

// (d >> 11) * 2^-53 for the ziggurat: the top 53 bits of the draw.
__device__ __forceinline__ double unit53_topbits(uint32_t lo, uint32_t hi) {
  return (double)hi * 0x1p-32 + (double)(lo >> 11) * 0x1p-53;
}

// Two binary16 values m 2^-11, m = h & 0x7FF, for the low and high halves h of w, packed;
// both halves at once with packed f16 arithmetic.  With r = m & 0x3FF and b = bit 10 of
// h: the half (r | 0x3800) encodes 1/2 + r 2^-11, which is m 2^-11 when b is set; when b
// is clear, 1/2 is taken off by one fused operation, the half (~h & 0x400) encoding 2^-14
// (and +0 when b is set) times -2^13.  Both cases are exact (m 2^-11 is a binary16 number),
// and m = 0 gives 1/2 - 1/2 = +0.  Three VALU instructions per word instead of seven for two
// conversions to f32, two products and a pack.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t half_pair_bits(uint32_t w) {
  // (w & 0x03FF03FF) | 0x38003800 and ~w & 0x04000400, each one v_bitop3 (truth tables
  // 0xEA = (a & b) | c and 0x0C = ~a & b)
  const uint32_t x = __builtin_amdgcn_bitop3_b32(w, 0x03FF03FFu, 0x38003800u, 0xEA);
  const uint32_t c = __builtin_amdgcn_bitop3_b32(w, 0x04000400u, 0u, 0x0C);
  f16x2 fx, fc;
  __builtin_memcpy(&fx, &x, 4);
  __builtin_memcpy(&fc, &c, 4);
  const f16x2 scale = {(_Float16)-8192.0f, (_Float16)-8192.0f};
  const f16x2 t = __builtin_elementwise_fma(fc, scale, fx);
  uint32_t bits;
  __builtin_memcpy(&bits, &t, 4);
  return bits;
}

// Four consecutive bits of `bits` starting at `shift`, one per byte (0 or 1).
__device__ __forceinline__ uint32_t nibble_to_bytes(uint32_t bits, int shift) {
  uint32_t nib = (bits >> shift) & 0xFu;
  return (nib * 0x00204081u) & 0x01010101u;  // bit j moves to bit 8j
}

// ---- cross-lane hand-off ----------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// The value held by the next lane of the wave (lane 63 receives 0; callers replace it or
// do not use it).  A wave-wide DPP shift (wave_shl:1, a gfx9-family VALU move) rather than
// ds_bpermute, which goes through LDS and costs a wait.  Every lane of the wave must
// execute this.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130 /* wave_shl:1 */, 0xF, 0xF, false);
}
__device__ __forceinline__ float from_next_lane(float v) { return __uint_as_float(from_next_lane(__float_as_uint(v))); }

// ---- substreams (tandem-sycl, "Design", §Normals: split(g) of sub(PURPOSE) of the key) --
// The host passes hkp = lowbias32(sub(key, P)); the substream of draw g has key
// split = word(hkp, g) and word j = word(lowbias32(split), j).
struct Substream {
  uint32_t hs;  // lowbias32 of the substream key
  uint32_t pos; // next 32-bit word
  __device__ __forceinline__ Substream(uint32_t hkp, uint32_t g) : hs(lowbias32(word(hkp, g))), pos(0) {}
  __device__ __forceinline__ uint32_t next32() { return word(hs, pos++); }
  __device__ __forceinline__ uint64_t next64() {
    uint32_t lo = word(hs, pos), hi = word(hs, pos + 1);
    pos += 2;
    return (uint64_t)lo | ((uint64_t)hi << 32);
  }
};

// Substream positions a rejection loop may consume before it stops; reaching it has
// probability below 2^-65536.  The result is then defined: the last value for bounded
// draws, NaN for normals.
constexpr uint32_t kSubstreamCap = 65536u;

// ---- Lemire multiply-shift with the exact threshold -----------------------------------
// t = (2^W - s) mod s precomputed on the host; a draw is accepted when the low half of
// x * s is at least t.
__device__ __forceinline__ uint32_t lemire32(uint32_t x, uint32_t s, uint32_t t, uint32_t hkp, uint32_t g) {
  uint64_t m = (uint64_t)x * s;
  if (__builtin_expect((uint32_t)m < t, 0)) {
    Substream ss(hkp, g);
    for (uint32_t j = 0; j < kSubstreamCap; ++j) {
      m = (uint64_t)ss.next32() * s;
      if ((uint32_t)m >= t) break;
    }
  }
  return (uint32_t)(m >> 32);
}

// 64 x 64 -> 128 multiply: returns the high half, low half in *lo.  When the bound fits
// 32 bits (kSmall) two 32 x 64 products suffice.
template <bool kSmall>
__device__ __forceinline__ uint64_t mul_hi_lo(uint64_t x, uint64_t s, uint64_t *lo) {
  if (kSmall) {
    uint64_t p0 = (uint64_t)(uint32_t)x * (uint32_t)s;
    uint64_t p1 = (x >> 32) * (uint32_t)s;
    uint64_t mid = p1 + (p0 >> 32);
    *lo = (mid << 32) | (uint32_t)p0;
    return mid >> 32;
  } else {
    *lo = x * s;
    return __umul64hi(x, s);
  }
}

template <bool kSmall>
__device__ __forceinline__ uint64_t lemire64(uint64_t x, uint64_t s, uint64_t t, uint32_t hkp, uint32_t g) {
  uint64_t lo;
  uint64_t hi = mul_hi_lo<kSmall>(x, s, &lo);
  if (__builtin_expect(lo < t, 0)) {
    Substream ss(hkp, g);
    for (uint32_t j = 0; j < kSubstreamCap; ++j) {
      hi = mul_hi_lo<kSmall>(ss.next64(), s, &lo);
      if (lo >= t) break;
    }
  }
  return hi;
}

// ---- Philox4x32-10 (Salmon et al., SC'11) ---------------------------------------------
struct U32x4 {
  uint32_t a, b, c, d;
};

// The block with counter (c0, c1, c2, c3) under key (k0, k1).
__device__ __forceinline__ U32x4 philox4x32_10_ctr(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                   uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-way xors as one gfx950 v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// The same rounds written with plain xors, for a block whose counter and key are the same
// across the wave: the compiler keeps it on the scalar unit (s_mul_hi_u32, s_mul_i32,
// s_xor_b32), where v_bitop3 would move it to the vector unit.
__device__ __forceinline__ U32x4 philox4x32_10_uniform(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                       uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// Primary block b: counter (lo32 b, hi32 b, 0, 0).
__device__ __forceinline__ U32x4 philox4x32_10(uint64_t block, uint32_t k0, uint32_t k1) {
  return philox4x32_10_ctr((uint32_t)block, (uint32_t)(block >> 32), 0u, 0u, k0, k1);
}

__device__ __forceinline__ uint32_t lane_of(const U32x4 &b, uint32_t j) {
  return j == 0 ? b.a : j == 1 ? b.b : j == 2 ? b.c : b.d;
}

// The Philox substream of draw i for purpose P: word j is lane j & 3 of the block with
// counter (lo32 i, hi32 i, P, j >> 2), disjoint from the primary blocks (counter words 2
// and 3 zero).  Nothing is computed until the first word is asked for, so a rejection
// loop that never runs costs nothing.
struct PhiloxSub {
  uint32_t k0, k1, c0, c1, purpose, pos;
  U32x4 blk;
  __device__ __forceinline__ PhiloxSub(uint32_t key0, uint32_t key1, uint64_t i, uint32_t p)
      : k0(key0), k1(key1), c0((uint32_t)i), c1((uint32_t)(i >> 32)), purpose(p), pos(0), blk{0, 0, 0, 0} {}
  __device__ __forceinline__ uint32_t next32() {
    if ((pos & 3u) == 0) blk = philox4x32_10_ctr(c0, c1, purpose, pos >> 2, k0, k1);
    return lane_of(blk, pos++ & 3u);
  }
  __device__ __forceinline__ uint64_t next64() {
    const uint32_t lo = next32(), hi = next32();
    return (uint64_t)lo | ((uint64_t)hi << 32);
  }
};

// Lemire's step with retries from a substream object (next32 / next64), for sources whose
// substream needs no set-up (Philox).
template <class Sub>
__device__ __forceinline__ uint32_t lemire32_sub(uint32_t x, uint32_t s, uint32_t t, Sub sub) {
  uint64_t m = (uint64_t)x * s;
  if (__builtin_expect((uint32_t)m < t, 0)) {
    for (uint32_t j = 0; j < kSubstreamCap; ++j) {
      m = (uint64_t)sub.next32() * s;
      if ((uint32_t)m >= t) break;
    }
  }
  return (uint32_t)(m >> 32);
}

template <bool kSmall, class Sub>
__device__ __forceinline__ uint64_t lemire64_sub(uint64_t x, uint64_t s, uint64_t t, Sub sub) {
  uint64_t lo;
  uint64_t hi = mul_hi_lo<kSmall>(x, s, &lo);
  if (__builtin_expect(lo < t, 0)) {
    for (uint32_t j = 0; j < kSubstreamCap; ++j) {
      hi = mul_hi_lo<kSmall>(sub.next64(), s, &lo);
      if (lo >= t) break;
    }
  }
  return hi;
}

// Four consecutive Philox words starting at word w0 (word offset w0 & 3 uniform across the
// launch, and the next lane's w0 four words on): the lane's own block plus, at unaligned
// offsets, the head of the next lane's.  Every lane of the wave must call this.
// With `overlap` the caller's lane 63 only feeds lane 62 (its own vector is the next wave's
// first), so it does not compute the next block.
__device__ __forceinline__ uint4 philox_words(uint64_t w0, uint32_t k0, uint32_t k1, bool overlap = false) {
  const uint64_t b = w0 >> 2;
  const uint32_t o = (uint32_t)(w0 & 3u);
  U32x4 B = philox4x32_10(b, k0, k1);
  if (o == 0) return make_uint4(B.a, B.b, B.c, B.d);
  uint32_t n0 = from_next_lane(B.a), n1 = from_next_lane(B.b), n2 = from_next_lane(B.c);
  if (!overlap && lane_id() == 63) {
    U32x4 N = philox4x32_10(b + 1, k0, k1);
    n0 = N.a; n1 = N.b; n2 = N.c;
  }
  if (o == 1) return make_uint4(B.b, B.c, B.d, n0);
  if (o == 2) return make_uint4(B.c, B.d, n0, n1);
  return make_uint4(B.d, n0, n1, n2);
}

__device__ __forceinline__ uint32_t philox_word(uint64_t w, uint32_t k0, uint32_t k1) {
  U32x4 B = philox4x32_10(w >> 2, k0, k1);
  const uint32_t o = (uint32_t)(w & 3u);
  return o == 0 ? B.a : o == 1 ? B.b : o == 2 ? B.c : B.d;
}

// ---- stores ----------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ void store16(void *p, uint4 v) {
  if (kNT) {
    u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4 *)p);
  } else {
    *(uint4 *)p = v;
  }
}

}  // namespace tk
