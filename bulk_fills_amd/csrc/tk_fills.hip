// tk_fills.hip -- streaming fill kernels: uniform, bounded, f32 normals, dropout,
// exponentials, Philox.
//
// One design serves every fill here.  The output is cut into whole 16-byte vectors from
// its first 4 KiB boundary; each lane computes the draws of one vector and writes it
// with one 16-byte store, so a wave64 store instruction covers 1 KiB of contiguous HBM.
// A work-group handles U consecutive runs of 256 vectors (4 KiB each; U = 1 by default,
// the shape that stores fastest), and the elements before the first 4 KiB boundary and
// after the last whole vector are written one at a time by block 0.
//
// Because every 32-bit word of the stream is its own counter, word-sized and wider draws
// never straddle a vector.  Sub-word draws (u8, u16, f16, bool), Box-Muller pairs at odd
// starts and Philox blocks at starts that are not a multiple of four straddle by at most
// one word, pair or block: that piece comes from the next lane through a DPP row shift
// (wave_shl:1).  The last lane of a wave computes its piece itself (sub-word draws, on
// the scalar unit), or takes it from the next wave through LDS (Box-Muller pairs,
// k_pair_tile; Philox blocks, k_philox_tile, which stages every block in LDS).  No extra
// HBM traffic.
#include "tk_device.h"
#include "tk_internal.h"
#include "tk_log.h"

namespace tk {

// ---------------------------------------------------------------------------------------
// Geometry and the generic kernel
// ---------------------------------------------------------------------------------------
template <class T>
struct FillBase {
  static constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte vector
  T *out;
  uint64_t start;  // draw of element 0
  uint64_t head;   // elements before the first 16-byte boundary
  uint64_t nvec;   // whole vectors
  uint32_t tail;   // elements after the last whole vector
  bool overlap;    // k_vec_fill_overlap: lane 63 of a wave only feeds lane 62
  // Launched as k_vec_line (no tile loop) when the grid covers the output: set by the
  // arithmetic-heavy ops, for which the loop's per-iteration compares and address updates
  // cost 4-11 % (MI355X, 2^28 elements: Box-Muller pairs 170 -> 152 us, one normal per
  // counter 227 -> 210, Philox f64 337 -> 300, u64 below 2^64 - 2 319 -> 308); the
  // store-bound fills measured the same or 1-2 % faster with the loop.
  static constexpr bool kLine = false;
  // Dynamic LDS per work-group, which caps the groups a compute unit holds (160 KiB of
  // LDS): the store-bound integer fills write faster with fewer groups in flight (MI355X,
  // 2^28 elements, alternating rounds: u32 155.5 -> 150.6 us and u64 308.5 -> 296.7 at
  // 32 KiB, five groups per compute unit; f64 299.4 -> 296.4 at 24 KiB), while the fills with
  // more arithmetic per store, or a load, lose time without the latency hiding of a full
  // compute unit (Box-Muller, Philox, exponentials, dropout: 0).
  static constexpr uint32_t kLdsPad = 0;
  __device__ __forceinline__ void *vec_ptr(uint64_t v) const { return (void *)(out + head + v * E); }
  __device__ __forceinline__ uint64_t vec_draw(uint64_t v) const { return start + head + v * E; }
};

// Vectors start at the output's first 4 KiB boundary, so that every work-group's tile of
// 256 vectors is 4 KiB-aligned; the elements before it (under 4 KiB) are written singly
// by block 0.  Measured on MI355X (u32, 2^28 elements, outputs 8 to 2056 bytes past a
// 4 KiB boundary): 156-158 us at every offset with 4 KiB alignment, 163-166 us with
// 1 KiB, 175-195 us with 128 bytes, and 213-220 us with vectors from the first 16-byte
// boundary (157 us on an aligned output).  f64: 300-307 against 350-380 us with 128 bytes.
constexpr uint64_t kGridAlign = 16 * kBlock;

template <class Base, class T>
static void set_geometry(Base &op, T *out, uint64_t start, uint64_t n) {
  constexpr uint64_t E = 16 / sizeof(T);
  uint64_t mis = (uint64_t)((uintptr_t)out & (kGridAlign - 1));
  uint64_t head = mis ? (kGridAlign - mis) / sizeof(T) : 0;
  if (head > n) head = n;
  op.out = out;
  op.start = start;
  op.head = head;
  op.nvec = (n - head) / E;
  op.tail = (uint32_t)(n - head - op.nvec * E);
}

// Writes the head elements (under 4 KiB of them) and the tail elements (fewer than 16)
// from block 0.
template <class Op>
__device__ __forceinline__ void write_edges(const Op &op) {
  for (uint64_t k = threadIdx.x; k < op.head; k += kBlock) op.out[k] = op.elem(k);
  if (threadIdx.x < op.tail) {
    const uint64_t k = op.head + op.nvec * Op::E + threadIdx.x;
    op.out[k] = op.elem(k);
  }
}

template <class Op, int U, bool kNT>
__global__ __launch_bounds__(kBlock) void k_vec_fill(Op op, uint64_t ntiles) {
  for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint64_t v0 = tile * (uint64_t)(kBlock * U) + threadIdx.x;
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = op.vec(v0 + (uint64_t)u * kBlock);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t v = v0 + (uint64_t)u * kBlock;
      if (v < op.nvec) store16<kNT>(op.vec_ptr(v), r[u]);
    }
  }
  if (blockIdx.x == 0) write_edges(op);
}

// One vector per lane, one tile per group, no loop: the grid covers the output.  Every
// lane computes its vector, also past the end, as in k_vec_fill: the ops' vectors may take
// a piece from the next lane or read lane 0 of the wave, so all 64 lanes must be active
// (kLine ops compute from counters only and read no memory).
template <class Op, bool kNT>
__global__ __launch_bounds__(kBlock) void k_vec_line(Op op) {
  const uint64_t v = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  const uint4 r = op.vec(v);
  if (v < op.nvec) store16<kNT>(op.vec_ptr(v), r);
  if (blockIdx.x == 0) write_edges(op);
}

template <class Op, int U>
static void launch_vec_u(const Op &op, hipStream_t stream) {
  const uint64_t per_tile = (uint64_t)kBlock * U;
  uint64_t ntiles = (op.nvec + per_tile - 1) / per_tile;
  uint64_t grid = ntiles ? ntiles : 1;
  if (U == 1 && Op::kLine && grid <= config().max_blocks && grid <= 0x7FFFFFFFull) {
    if (config().nt_stores)
      hipLaunchKernelGGL((k_vec_line<Op, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
    else
      hipLaunchKernelGGL((k_vec_line<Op, false>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
    return;
  }
  if (grid > config().max_blocks) grid = config().max_blocks;
  if (grid > 0x7FFFFFFFull) grid = 0x7FFFFFFFull;
  if (config().nt_stores)
    hipLaunchKernelGGL((k_vec_fill<Op, U, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op, ntiles);
  else
    hipLaunchKernelGGL((k_vec_fill<Op, U, false>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op, ntiles);
}

// Philox fills at word offsets that are not a multiple of four, whose vector needs the head
// of the next lane's block: each wave stores 63 vectors, and its lane 63 computes the next
// wave's first block only to hand its head to lane 62.  That costs 1/64 more arithmetic
// instead of a divergent second block in lane 63 of every wave, and every store stays one
// 16-byte vector.  Measured on MI355X (2^28 elements): Philox u32 at start 1 or 2 from
// ~224 to ~205 us, the Philox normal f32 from ~260 to ~190-205 us.  For lowbias32
// Box-Muller pairs at odd starts it measured no better than the divergent pair (~208 us
// either way): a wave span of 1008 bytes alone costs that much; those take the pair tile
// kernel below.
template <class Op, bool kNT>
__global__ __launch_bounds__(kBlock) void k_vec_fill_overlap(Op op) {
  const uint64_t wave = (uint64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const uint32_t lane = (uint32_t)lane_id();
  const uint64_t v = wave * 63 + lane;
  const uint4 r = op.vec(v);
  if (lane < 63 && v < op.nvec) store16<kNT>(op.vec_ptr(v), r);
  if (blockIdx.x == 0) write_edges(op);
}

template <class Op>
static tk_status launch_vec_overlap(Op op, hipStream_t stream) {
  op.overlap = true;
  const uint64_t waves = (op.nvec + 62) / 63;
  uint64_t grid = (waves + kBlock / 64 - 1) / (kBlock / 64);
  if (grid == 0) grid = 1;
  if (grid > 0x7FFFFFFFull) return TK_EINVAL;
  if (config().nt_stores)
    hipLaunchKernelGGL((k_vec_fill_overlap<Op, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  else
    hipLaunchKernelGGL((k_vec_fill_overlap<Op, false>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  return launch_status();
}

// Philox fills at word offsets o = 1..3 staged through LDS (the tile kernel).  Each
// work-group writes one 4 KiB tile, as the aligned fills do: every lane computes its own
// block-aligned Philox block, the one the first word of its vector falls in, and writes it
// to LDS; the block after the tile, whose counter is the same for the whole group, is
// computed once on the scalar unit by the last wave.  After one barrier each lane reads
// its four words at word offset o from LDS and stores one 16-byte vector.  The shape of the
// stores is that of the aligned fills (whole 4 KiB tiles per group, 1 KiB per wave).
template <class Op, bool kNT>
__global__ __launch_bounds__(kBlock) void k_philox_tile(Op op) {
  __shared__ uint4 blk[kBlock + 1];
  const uint64_t v0 = (uint64_t)blockIdx.x * kBlock;
  const uint64_t wt = op.word0(v0);  // first word of the tile: 4 (b0 + lane) + o for each lane
  const uint64_t b0 = wt >> 2;
  const U32x4 B = philox4x32_10(b0 + threadIdx.x, op.k0, op.k1);
  blk[threadIdx.x] = make_uint4(B.a, B.b, B.c, B.d);
  if ((uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == kBlock / 64 - 1) {
    const uint64_t bn = b0 + kBlock;  // uniform counter: scalar unit
    const U32x4 N = philox4x32_10_uniform((uint32_t)bn, (uint32_t)(bn >> 32), 0u, 0u, op.k0, op.k1);
    if (lane_id() == 0) blk[kBlock] = make_uint4(N.a, N.b, N.c, N.d);
  }
  __syncthreads();
  const uint32_t *wp = (const uint32_t *)blk + 4 * threadIdx.x + (uint32_t)(wt & 3u);
  const uint64_t v = v0 + threadIdx.x;
  const uint4 r = op.from_words(v, make_uint4(wp[0], wp[1], wp[2], wp[3]));
  if (v < op.nvec) store16<kNT>(op.vec_ptr(v), r);
  if (blockIdx.x == 0) write_edges(op);
}

template <class Op>
static tk_status launch_philox_tile(const Op &op, hipStream_t stream) {
  uint64_t grid = (op.nvec + kBlock - 1) / kBlock;
  if (grid == 0) grid = 1;
  if (grid > 0x7FFFFFFFull) return TK_EINVAL;
  if (config().nt_stores)
    hipLaunchKernelGGL((k_philox_tile<Op, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  else
    hipLaunchKernelGGL((k_philox_tile<Op, false>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  return launch_status();
}

// Box-Muller pairs at odd start draws (lowbias32): a vector is sin of pair c0, pair c0+1
// and cos of pair c0+2, whose cosine is the next lane's first value.  Lanes take it from
// their neighbour; lane 63 of a wave takes lane 0's of the next wave through LDS; and the
// last wave computes the first pair of the next tile once (its counter is the same for the
// whole wave: the hashes run on the scalar unit, the cosine's arithmetic once per group
// instead of once per wave).  One barrier per group; stores as in the aligned fills.
template <class Op, bool kNT>
__global__ __launch_bounds__(kBlock) void k_pair_tile(Op op) {
  constexpr uint32_t kWaves = kBlock / 64;
  __shared__ float first[kWaves + 1];
  const uint64_t v = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  const uint32_t c0 = (uint32_t)(op.vec_draw(v) >> 1);
  float a, b, c, d;
  op.pair(c0, &a, &b);
  op.pair(c0 + 1u, &c, &d);
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lane_id() == 0) first[wave] = a;
  if (wave == kWaves - 1) {
    const uint32_t cn = (uint32_t)__builtin_amdgcn_readfirstlane(c0) + 128u;  // 64 lanes, 2 pairs each
    float en, s_unused;
    op.pair(cn, &en, &s_unused);
    if (lane_id() == 0) first[kWaves] = en;
  }
  float e = from_next_lane(a);
  __syncthreads();
  if (lane_id() == 63) e = first[wave + 1];
  if (v < op.nvec)
    store16<kNT>(op.vec_ptr(v), make_uint4(__float_as_uint(b), __float_as_uint(c), __float_as_uint(d), __float_as_uint(e)));
  if (blockIdx.x == 0) write_edges(op);
}

template <class Op>
static tk_status launch_pair_tile(const Op &op, hipStream_t stream) {
  uint64_t grid = (op.nvec + kBlock - 1) / kBlock;
  if (grid == 0) grid = 1;
  if (grid > 0x7FFFFFFFull) return TK_EINVAL;
  if (config().nt_stores)
    hipLaunchKernelGGL((k_pair_tile<Op, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  else
    hipLaunchKernelGGL((k_pair_tile<Op, false>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  return launch_status();
}

// One vector per lane and one 4 KiB tile per work-group over a grid as large as the
// output measured fastest for streaming stores on MI355X (more vectors per lane or a
// persistent grid lowered the store rate); TK_UNROLL=2|4 selects the alternatives.
template <class Op>
static tk_status launch_vec(const Op &op, hipStream_t stream) {
  switch (config().unroll) {
    case 2: launch_vec_u<Op, 2>(op, stream); break;
    case 4: launch_vec_u<Op, 4>(op, stream); break;
    default: launch_vec_u<Op, 1>(op, stream); break;
  }
  return launch_status();
}

// The same launch with non-temporal 16-byte stores whatever TK_STORE says: for dropout,
// whose input is read with non-temporal loads.  A 1 GiB scaled copy measured 6.2 TB/s moved
// with plain loads and stores, 6.5 with non-temporal loads and 6.6 with both; the 2^28
// dropout went from ~346 to ~328 us (out of place) and from ~358 to ~324 us (in place).
template <class Op>
static tk_status launch_vec_nt(const Op &op, hipStream_t stream) {
  uint64_t ntiles = (op.nvec + kBlock - 1) / kBlock;
  uint64_t grid = ntiles ? ntiles : 1;
  if (grid > config().max_blocks) grid = config().max_blocks;
  if (grid > 0x7FFFFFFFull) grid = 0x7FFFFFFFull;
  hipLaunchKernelGGL((k_vec_fill<Op, 1, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op, ntiles);
  return launch_status();
}

__device__ __forceinline__ uint4 u4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) { return make_uint4(a, b, c, d); }
__device__ __forceinline__ uint32_t lo32(uint64_t x) { return (uint32_t)x; }
__device__ __forceinline__ uint32_t hi32(uint64_t x) { return (uint32_t)(x >> 32); }

// ---------------------------------------------------------------------------------------
// Constant fill: no generator, only the store path.  The same geometry, grid and 16-byte
// stores as every streaming fill, so its rate is the ceiling those fills are measured
// against.
// ---------------------------------------------------------------------------------------
// `work` (a tunable, 0 by default) puts a chain of that many dependent integer steps before
// each lane's store: the fills store after some arithmetic, and the rate of stores spaced
// that way is part of what the ceiling has to cover.
struct OpConst : FillBase<uint32_t> {
  uint32_t value;
  uint32_t work;
  __device__ __forceinline__ uint32_t elem(uint64_t) const { return value; }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    if (work) {
      uint32_t x = (uint32_t)v;
      for (uint32_t i = 0; i < work; ++i) x = x * 0x01000193u + i;
      __asm__ volatile("" ::"v"(x));  // keeps the chain; the stored value does not depend on it
    }
    return u4(value, value, value, value);
  }
};

// ---------------------------------------------------------------------------------------
// Uniform fills
// ---------------------------------------------------------------------------------------
// u32 / f32: draw i is word i.
template <bool kFloat>
struct OpWord32 : FillBase<uint32_t> {
  static constexpr uint32_t kLdsPad = 32768;
  uint32_t hk;
  __device__ __forceinline__ uint32_t xf(uint32_t w) const { return kFloat ? __float_as_uint(unit23(w)) : w; }
  __device__ __forceinline__ uint32_t elem(uint64_t k) const { return xf(word(hk, (uint32_t)(start + k))); }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint32_t c = (uint32_t)vec_draw(v);
    return u4(xf(word(hk, c)), xf(word(hk, c + 1)), xf(word(hk, c + 2)), xf(word(hk, c + 3)));
  }
};

// u64 / f64: draw i is words 2i (low) and 2i+1 (high).
template <bool kFloat>
struct OpWord64 : FillBase<uint64_t> {
  static constexpr uint32_t kLdsPad = kFloat ? 24576 : 32768;
  uint32_t hk;
  __device__ __forceinline__ uint64_t xf(uint32_t lo, uint32_t hi) const {
    if (kFloat) return (uint64_t)__double_as_longlong(unit53_lowbits(lo, hi));
    return (uint64_t)lo | ((uint64_t)hi << 32);
  }
  __device__ __forceinline__ uint64_t elem(uint64_t k) const {
    const uint32_t c = 2u * (uint32_t)(start + k);
    return xf(word(hk, c), word(hk, c + 1));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint32_t c = 2u * (uint32_t)vec_draw(v);
    uint64_t a = xf(word(hk, c), word(hk, c + 1));
    uint64_t b = xf(word(hk, c + 2), word(hk, c + 3));
    return u4(lo32(a), hi32(a), lo32(b), hi32(b));
  }
};

// Four consecutive stream words starting `shift` bytes into word w0: lane-local words
// w0..w0+3, the fifth from the next lane.  The last lane's fifth word is the next wave's
// first, w0 of lane 0 plus 256: its counter is the same for the whole wave, so it is hashed
// once per wave on the scalar unit (about eight scalar instructions) instead of by every
// lane.  All 64 lanes must be active (lane 0's w0 is read with readfirstlane).  `shift` is
// uniform across the launch.
__device__ __forceinline__ uint4 words_at_byte(uint32_t hk, uint32_t w0, uint32_t shift) {
  uint32_t a0 = word(hk, w0), a1 = word(hk, w0 + 1), a2 = word(hk, w0 + 2), a3 = word(hk, w0 + 3);
  if (shift == 0) return u4(a0, a1, a2, a3);
  const uint32_t next_wave = word(hk, (uint32_t)__builtin_amdgcn_readfirstlane(w0) + 256u);
  uint32_t a4 = from_next_lane(a0);
  if (lane_id() == 63) a4 = next_wave;
  return u4(__builtin_amdgcn_alignbyte(a1, a0, shift), __builtin_amdgcn_alignbyte(a2, a1, shift),
            __builtin_amdgcn_alignbyte(a3, a2, shift), __builtin_amdgcn_alignbyte(a4, a3, shift));
}

// u16 / f16 bits: draw i is half i&1 of word i>>1.
template <bool kHalf>
struct OpSub16 : FillBase<uint16_t> {
  static constexpr uint32_t kLdsPad = kHalf ? 0 : 24576;  // f16: 77.9 -> 82.0 us with a cap
  uint32_t hk;
  __device__ __forceinline__ uint16_t elem(uint64_t k) const {
    const uint64_t i = start + k;
    uint32_t h = word(hk, (uint32_t)(i >> 1)) >> (16u * (uint32_t)(i & 1u));
    return (uint16_t)(kHalf ? half_pair_bits(h) : h);
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint64_t i0 = vec_draw(v);
    uint4 w = words_at_byte(hk, (uint32_t)(i0 >> 1), 2u * (uint32_t)(i0 & 1u));
    if (kHalf) w = u4(half_pair_bits(w.x), half_pair_bits(w.y), half_pair_bits(w.z), half_pair_bits(w.w));
    return w;
  }
};

// u8: draw i is byte i&3 of word i>>2.
struct OpU8 : FillBase<uint8_t> {
  uint32_t hk;
  __device__ __forceinline__ uint8_t elem(uint64_t k) const {
    const uint64_t i = start + k;
    return (uint8_t)(word(hk, (uint32_t)(i >> 2)) >> (8u * (uint32_t)(i & 3u)));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint64_t i0 = vec_draw(v);
    return words_at_byte(hk, (uint32_t)(i0 >> 2), (uint32_t)(i0 & 3u));
  }
};

// bool: draw i is bit i&31 of word i>>5, one byte 0/1 per bit.
struct OpBool : FillBase<uint8_t> {
  uint32_t hk;
  __device__ __forceinline__ uint8_t elem(uint64_t k) const {
    const uint64_t i = start + k;
    return (uint8_t)((word(hk, (uint32_t)(i >> 5)) >> (uint32_t)(i & 31u)) & 1u);
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint64_t b0 = vec_draw(v);
    const uint32_t wi = (uint32_t)(b0 >> 5);
    const uint32_t lo = word(hk, wi), hi = word(hk, wi + 1);
    const uint32_t bits = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(b0 & 31u));
    return u4(nibble_to_bytes(bits, 0), nibble_to_bytes(bits, 4), nibble_to_bytes(bits, 8), nibble_to_bytes(bits, 12));
  }
};

// ---------------------------------------------------------------------------------------
// Bounded integers (Lemire, exact threshold; rejected draws continue on the substream)
// ---------------------------------------------------------------------------------------
struct Below32Params {
  uint32_t hk, hkp, s, t;
  int64_t low;
};

// u32 / i32 out, one word per element.
template <class T>
struct OpBelow32 : FillBase<T> {
  static constexpr uint32_t kLdsPad = 32768;
  Below32Params p;
  __device__ __forceinline__ T elem(uint64_t k) const {
    const uint32_t i = (uint32_t)(this->start + k);
    return (T)((uint32_t)p.low + lemire32(word(p.hk, i), p.s, p.t, p.hkp, i));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint32_t i = (uint32_t)this->vec_draw(v);
    uint32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (uint32_t)p.low + lemire32(word(p.hk, i + j), p.s, p.t, p.hkp, i + j);
    return u4(r[0], r[1], r[2], r[3]);
  }
};

// i64 out from one word per element: each 16-byte vector holds two elements.
struct OpBelow32To64 : FillBase<int64_t> {
  static constexpr uint32_t kLdsPad = 32768;
  Below32Params p;
  __device__ __forceinline__ int64_t elem(uint64_t k) const {
    const uint32_t i = (uint32_t)(start + k);
    return p.low + (int64_t)lemire32(word(p.hk, i), p.s, p.t, p.hkp, i);
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint32_t i = (uint32_t)vec_draw(v);
    uint64_t a = (uint64_t)(p.low + (int64_t)lemire32(word(p.hk, i), p.s, p.t, p.hkp, i));
    uint64_t b = (uint64_t)(p.low + (int64_t)lemire32(word(p.hk, i + 1), p.s, p.t, p.hkp, i + 1));
    return u4(lo32(a), hi32(a), lo32(b), hi32(b));
  }
};

// u64 / i64 out from one 64-bit draw per element.
template <class T, bool kSmall>
struct OpBelow64 : FillBase<T> {
  static constexpr bool kLine = !kSmall;  // the 64-bit products of bounds above 2^32
  static constexpr uint32_t kLdsPad = kSmall ? 32768 : 0;
  uint32_t hk, hkp;
  uint64_t s, t;
  int64_t low;
  __device__ __forceinline__ uint64_t one(uint32_t i) const {
    const uint32_t c = 2u * i;
    uint64_t x = (uint64_t)word(hk, c) | ((uint64_t)word(hk, c + 1) << 32);
    return (uint64_t)low + lemire64<kSmall>(x, s, t, hkp, i);
  }
  __device__ __forceinline__ T elem(uint64_t k) const { return (T)one((uint32_t)(this->start + k)); }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint32_t i = (uint32_t)this->vec_draw(v);
    uint64_t a = one(i), b = one(i + 1);
    return u4(lo32(a), hi32(a), lo32(b), hi32(b));
  }
};

// ---------------------------------------------------------------------------------------
// f32 normal: Box-Muller pairs (draw i belongs to pair i >> 1; even i cos, odd i sin)
// ---------------------------------------------------------------------------------------
template <bool kHalfTurn>
struct OpNormalF32 : FillBase<float> {
  static constexpr bool kLine = true;
  uint32_t hk;
  // Pair c is the public API's tk_randn2_f32 (or its half-turn form): r = sqrt(-2 ln(1 - u1))
  // with the hardware base-2 logarithm (ln x = ln 2 * log2 x) and square root; cos and sin
  // of 2 pi t with the hardware sine and cosine, which take their argument in turns, so t
  // in [-1/2, 1/2) goes in unscaled.  Measured on MI355X over every 2^-23 grid value:
  // radius error <= 4.7e-7, sine and cosine error <= 1.3e-7, so |error| <= 1.2e-6 for
  // |x| < 5.65.
  __device__ __forceinline__ void pair(uint32_t c, float *cs, float *sn) const {
    if (kHalfTurn) tk_box_muller_half_turn_f32(word(hk, 2u * c), word(hk, 2u * c + 1u), cs, sn);
    else tk_randn2_f32(hk, c, cs, sn);
  }
  __device__ __forceinline__ float elem(uint64_t k) const {
    const uint64_t i = start + k;
    float c, s;
    pair((uint32_t)(i >> 1), &c, &s);
    return (i & 1u) ? s : c;
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint64_t i0 = vec_draw(v);
    const uint32_t c0 = (uint32_t)(i0 >> 1);
    float a, b, c, d;
    pair(c0, &a, &b);
    pair(c0 + 1, &c, &d);
    if ((i0 & 1u) == 0) return u4(__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d));
    // Odd start: the vector is sin(c0), pair c0+1, cos(c0+2); cos(c0+2) is the next
    // lane's first value.  The last lane's is the next wave's first pair, lane 0's c0 plus
    // 128, the same for the whole wave: its two words are hashed on the scalar unit and
    // only the cosine's arithmetic runs on the vector unit, once for the wave (all 64
    // lanes must be active: lane 0's c0 is read with readfirstlane).
    float e = from_next_lane(a);
    if (!overlap) {
      const uint32_t cn = (uint32_t)__builtin_amdgcn_readfirstlane(c0) + 128u;
      float en, s_unused;
      pair(cn, &en, &s_unused);
      if (lane_id() == 63) e = en;
    }
    return u4(__float_as_uint(b), __float_as_uint(c), __float_as_uint(d), __float_as_uint(e));
  }
};

// One normal per counter (Phobos, §randn): element i is the cosine of pair i.
struct OpRandnF32 : FillBase<float> {
  static constexpr bool kLine = true;
  uint32_t hk;
  __device__ __forceinline__ float elem(uint64_t k) const { return tk_randn_f32(hk, (uint32_t)(start + k)); }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint32_t c = (uint32_t)vec_draw(v);
    return u4(__float_as_uint(tk_randn_f32(hk, c)), __float_as_uint(tk_randn_f32(hk, c + 1)),
              __float_as_uint(tk_randn_f32(hk, c + 2)), __float_as_uint(tk_randn_f32(hk, c + 3)));
  }
};

// ---------------------------------------------------------------------------------------
// Exponentials: x = -ln(1 - u), +0 at u = 0, by inversion of the uniform draw.  1 - u is
// exact for both types and the logarithms are tk_log.h's: the f64 one within 0.502 ulp, the
// f32 one rounded once to the correctly rounded f32 at every point of its 2^-24 grid.
// ---------------------------------------------------------------------------------------
// f64: u = (d & (2^53 - 1)) 2^-53 of the 64-bit draw.
struct OpExpF64 : FillBase<uint64_t> {
  using Entry = LogEntryWide;  // the LDS copy; the table itself holds LogEntryD
  static constexpr bool kWiden = true;
  static constexpr int kEntries = TK_LOGD_ENTRIES;
  __device__ static const LogEntryD *table() { return kLogTableD; }
  uint32_t hk;
  __device__ __forceinline__ uint64_t elem(uint64_t k) const {
    const uint32_t c = 2u * (uint32_t)(start + k);
    return (uint64_t)__double_as_longlong(neg_ln_draw53(word(hk, c), word(hk, c + 1), kLogTableD));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v, const Entry *tab) const {
    const uint32_t c = 2u * (uint32_t)vec_draw(v);
    const uint64_t a = (uint64_t)__double_as_longlong(neg_ln_draw53(word(hk, c), word(hk, c + 1), tab));
    const uint64_t b = (uint64_t)__double_as_longlong(neg_ln_draw53(word(hk, c + 2), word(hk, c + 3), tab));
    return u4(lo32(a), hi32(a), lo32(b), hi32(b));
  }
};

// f32: u = (w & 0xFFFFFF) 2^-24.
struct OpExpF32 : FillBase<uint32_t> {
  using Entry = LogEntryF;
  static constexpr bool kWiden = false;
  static constexpr int kEntries = TK_LOGF_ENTRIES;
  __device__ static const Entry *table() { return kLogTableF; }
  uint32_t hk;
  __device__ __forceinline__ uint32_t one(uint32_t w, const LogEntryF *tab) const {
    return __float_as_uint(neg_ln_grid24_f32(w & 0xFFFFFFu, tab));
  }
  __device__ __forceinline__ uint32_t elem(uint64_t k) const { return one(word(hk, (uint32_t)(start + k)), kLogTableF); }
  __device__ __forceinline__ uint4 vec(uint64_t v, const LogEntryF *tab) const {
    const uint32_t c = (uint32_t)vec_draw(v);
    return u4(one(word(hk, c), tab), one(word(hk, c + 1), tab), one(word(hk, c + 2), tab), one(word(hk, c + 3), tab));
  }
};

// Exponential fills: T 4 KiB tiles per work-group after copying the fill's 4 KiB logarithm
// table to LDS (16-byte loads, all issued before the LDS writes; the f64 fill widens each
// entry to three doubles on the way), so the per-element table reads are ds_reads and not
// L1 gathers through the texture addresser.
template <class Op, int T, bool kNT>
__global__ __launch_bounds__(kBlock) void k_exp_fill(Op op) {
  using Entry = typename Op::Entry;
  __shared__ __align__(16) Entry tab[Op::kEntries];
  if constexpr (Op::kWiden) {  // one entry per lane, widened to whole doubles
    static_assert(Op::kEntries == kBlock, "one table entry per lane");
    const LogEntryD e = Op::table()[threadIdx.x];
    tab[threadIdx.x] = Entry{e.l_hi, log_m(e), log_l_lo(e)};
  } else {
    constexpr int kPieces = (int)(sizeof(Entry) * Op::kEntries / 16);
    constexpr int kPer = (kPieces + kBlock - 1) / kBlock;
    static_assert(sizeof(Entry) * Op::kEntries % 16 == 0, "the table copies in 16-byte pieces");
    uint4 piece[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = (int)threadIdx.x + r * kBlock;
      if (i < kPieces) piece[r] = ((const uint4 *)Op::table())[i];
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = (int)threadIdx.x + r * kBlock;
      if (i < kPieces) ((uint4 *)tab)[i] = piece[r];
    }
  }
  __syncthreads();
  const uint64_t v0 = (uint64_t)blockIdx.x * T * kBlock + threadIdx.x;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint64_t v = v0 + (uint64_t)t * kBlock;
    const uint4 r = op.vec(v, tab);
    if (v < op.nvec) store16<kNT>(op.vec_ptr(v), r);
  }
  if (blockIdx.x == 0) write_edges(op);
}

template <class Op, int T>
static tk_status launch_exp_t(const Op &op, hipStream_t stream) {
  const uint64_t per = (uint64_t)kBlock * T;
  uint64_t grid = (op.nvec + per - 1) / per;
  if (grid == 0) grid = 1;
  if (grid > 0x7FFFFFFFull) return TK_EINVAL;
  if (config().nt_stores)
    hipLaunchKernelGGL((k_exp_fill<Op, T, true>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  else
    hipLaunchKernelGGL((k_exp_fill<Op, T, false>), dim3((uint32_t)grid), dim3(kBlock), lds_pad<Op>(), stream, op);
  return launch_status();
}

template <class Op, class T>
static tk_status run_exp(Op op, T *out, uint64_t start, uint64_t n, hipStream_t stream) {
  set_geometry(op, out, start, n);
  switch (config().exp_tiles) {
    case 1: return launch_exp_t<Op, 1>(op, stream);
    case 4: return launch_exp_t<Op, 4>(op, stream);
    default: return launch_exp_t<Op, 2>(op, stream);
  }
}

// ---------------------------------------------------------------------------------------
// Fused dropout: y = u >= p ? x / (1 - p) : +0 (IEEE f32 division), optional mask bytes
// ---------------------------------------------------------------------------------------
struct OpDropout : FillBase<float> {
  const float *x;
  uint8_t *mask;
  uint32_t hk;
  float p, q;
  bool x_vec;      // x is 16-byte aligned where y is
  bool mask_word;  // mask is 4-byte aligned where y is 16-byte aligned
  __device__ __forceinline__ float elem(uint64_t k) const {
    const bool keep = tk_dropout_keep(p, hk, (uint32_t)(start + k));
    if (mask) mask[k] = (uint8_t)keep;
    return keep ? __fdiv_rn(x[k], q) : 0.0f;
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    if (v >= nvec) return u4(0, 0, 0, 0);  // never read x past the end
    const uint64_t k0 = head + 4 * v;
    float xv[4];
    if (x_vec) {  // x is read once: a non-temporal load (streams past the caches)
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4 t = __builtin_nontemporal_load((const f32x4 *)(x + k0));
      xv[0] = t.x; xv[1] = t.y; xv[2] = t.z; xv[3] = t.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = x[k0 + j];
    }
    const uint32_t c = (uint32_t)(start + k0);
    uint32_t y[4], m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool keep = tk_dropout_keep(p, hk, c + j);
      y[j] = keep ? __float_as_uint(__fdiv_rn(xv[j], q)) : 0u;
      m |= (uint32_t)keep << (8 * j);
    }
    if (mask) {
      if (mask_word) *(uint32_t *)(mask + k0) = m;
      else
#pragma unroll
        for (int j = 0; j < 4; ++j) mask[k0 + j] = (uint8_t)(m >> (8 * j));
    }
    return u4(y[0], y[1], y[2], y[3]);
  }
};

// ---------------------------------------------------------------------------------------
// Philox4x32-10 word source
// ---------------------------------------------------------------------------------------
// Every Philox streaming op builds vector v from the four consecutive words at word0(v)
// (four words per vector: 32-bit draws one word each, 64-bit draws two) with
// from_words(v, w); vec(v) computes those words in registers, the tile kernel stages them
// through LDS.
template <bool kFloat>
struct OpPhilox32 : FillBase<uint32_t> {
  uint32_t k0, k1;
  __device__ __forceinline__ uint32_t xf(uint32_t w) const { return kFloat ? __float_as_uint(unit23(w)) : w; }
  __device__ __forceinline__ uint32_t elem(uint64_t k) const { return xf(philox_word(start + k, k0, k1)); }
  __device__ __forceinline__ uint64_t word0(uint64_t v) const { return vec_draw(v); }
  __device__ __forceinline__ uint4 from_words(uint64_t, uint4 w) const { return u4(xf(w.x), xf(w.y), xf(w.z), xf(w.w)); }
  __device__ __forceinline__ uint4 vec(uint64_t v) const { return from_words(v, philox_words(word0(v), k0, k1, overlap)); }
};

template <bool kFloat>
struct OpPhilox64 : FillBase<uint64_t> {
  static constexpr bool kLine = true;
  uint32_t k0, k1;
  __device__ __forceinline__ uint64_t xf(uint32_t lo, uint32_t hi) const {
    if (kFloat) return (uint64_t)__double_as_longlong(unit53_lowbits(lo, hi));
    return (uint64_t)lo | ((uint64_t)hi << 32);
  }
  __device__ __forceinline__ uint64_t elem(uint64_t k) const {
    const uint64_t w = 2 * (start + k);
    return xf(philox_word(w, k0, k1), philox_word(w + 1, k0, k1));
  }
  __device__ __forceinline__ uint64_t word0(uint64_t v) const { return 2 * vec_draw(v); }
  __device__ __forceinline__ uint4 from_words(uint64_t, uint4 w) const {
    const uint64_t a = xf(w.x, w.y), b = xf(w.z, w.w);
    return u4(lo32(a), hi32(a), lo32(b), hi32(b));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const { return from_words(v, philox_words(word0(v), k0, k1, overlap)); }
};

// ---------------------------------------------------------------------------------------
// Philox variants of the bounded and normal fills: the definitions above over Philox
// words; a rejected draw i continues on PhiloxSub(i, purpose)
// ---------------------------------------------------------------------------------------
struct OpPhiloxBelow32 : FillBase<uint32_t> {
  uint32_t k0, k1, s, t;
  __device__ __forceinline__ uint32_t one(uint32_t w, uint64_t i) const {
    return lemire32_sub(w, s, t, PhiloxSub(k0, k1, i, kPurposeBelow32));
  }
  __device__ __forceinline__ uint32_t elem(uint64_t k) const { return one(philox_word(start + k, k0, k1), start + k); }
  __device__ __forceinline__ uint64_t word0(uint64_t v) const { return vec_draw(v); }
  __device__ __forceinline__ uint4 from_words(uint64_t v, uint4 w) const {
    const uint64_t i = vec_draw(v);
    return u4(one(w.x, i), one(w.y, i + 1), one(w.z, i + 2), one(w.w, i + 3));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const { return from_words(v, philox_words(word0(v), k0, k1, overlap)); }
};

template <bool kSmall>
struct OpPhiloxBelow64 : FillBase<uint64_t> {
  uint32_t k0, k1;
  uint64_t s, t;
  __device__ __forceinline__ uint64_t one(uint32_t lo, uint32_t hi, uint64_t i) const {
    return lemire64_sub<kSmall>((uint64_t)lo | ((uint64_t)hi << 32), s, t, PhiloxSub(k0, k1, i, kPurposeBelow64));
  }
  __device__ __forceinline__ uint64_t elem(uint64_t k) const {
    const uint64_t i = start + k;
    return one(philox_word(2 * i, k0, k1), philox_word(2 * i + 1, k0, k1), i);
  }
  __device__ __forceinline__ uint64_t word0(uint64_t v) const { return 2 * vec_draw(v); }
  __device__ __forceinline__ uint4 from_words(uint64_t v, uint4 w) const {
    const uint64_t i = vec_draw(v);
    const uint64_t a = one(w.x, w.y, i), b = one(w.z, w.w, i + 1);
    return u4(lo32(a), hi32(a), lo32(b), hi32(b));
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const { return from_words(v, philox_words(word0(v), k0, k1, overlap)); }
};

// Box-Muller pairs over Philox words (pair c: words 2c and 2c+1), laid out as OpNormalF32.
struct OpPhiloxNormalF32 : FillBase<float> {
  static constexpr bool kLine = true;
  uint32_t k0, k1;
  __device__ __forceinline__ void pair(uint64_t c, float *cs, float *sn) const {
    tk_box_muller_f32(philox_word(2 * c, k0, k1), philox_word(2 * c + 1, k0, k1), cs, sn);
  }
  __device__ __forceinline__ float elem(uint64_t k) const {
    const uint64_t i = start + k;
    float c, s;
    pair(i >> 1, &c, &s);
    return (i & 1u) ? s : c;
  }
  __device__ __forceinline__ uint4 vec(uint64_t v) const {
    const uint64_t i0 = vec_draw(v);
    const uint64_t c0 = i0 >> 1;
    const uint4 w = philox_words(2 * c0, k0, k1, overlap);  // pairs c0 and c0 + 1 (word offset 0 or 2, uniform)
    float a, b, c, d;
    tk_box_muller_f32(w.x, w.y, &a, &b);
    tk_box_muller_f32(w.z, w.w, &c, &d);
    if ((i0 & 1u) == 0) return u4(__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d));
    float e = from_next_lane(a);  // the next lane's first pair is c0 + 2
    if (!overlap && lane_id() == 63) {
      float s_unused;
      pair(c0 + 2, &e, &s_unused);
    }
    return u4(__float_as_uint(b), __float_as_uint(c), __float_as_uint(d), __float_as_uint(e));
  }
};

}  // namespace tk

// =======================================================================================
// C ABI entry points
// =======================================================================================
using namespace tk;

namespace {

// Draws needed by a fill of n elements from `start` must all be <= dmax.
tk_status check_draws(uint64_t start, uint64_t n, uint64_t dmax) {
  if (start > dmax || n - 1 > dmax - start) return TK_ERANGE;
  return TK_OK;
}

template <class T>
bool elem_aligned(const T *p) { return ((uintptr_t)p % sizeof(T)) == 0; }

constexpr uint64_t kMaxW32 = 0xFFFFFFFFull;        // one word per draw
constexpr uint64_t kMaxW64 = 0x7FFFFFFFull;        // two words per draw
constexpr uint64_t kMaxU16 = 0x1FFFFFFFFull;       // half a word per draw
constexpr uint64_t kMaxU8 = 0x3FFFFFFFFull;        // a quarter word per draw
constexpr uint64_t kMaxBool = 0x1FFFFFFFFFull;     // a bit per draw
constexpr uint64_t kMaxPhilox64 = 0x7FFFFFFFFFFFFFFFull;

#define TK_PRECHECK(ptr, dmax)                         \
  do {                                                 \
    if (n == 0) return TK_OK;                          \
    if (!(ptr) || !elem_aligned(ptr)) return TK_EINVAL; \
    tk_status st_ = check_draws(start_draw, n, (dmax)); \
    if (st_ != TK_OK) return st_;                      \
  } while (0)

template <class Op, class T>
tk_status run_simple(Op op, T *out, uint64_t start, uint64_t n, hipStream_t stream) {
  set_geometry(op, out, start, n);
  return launch_vec(op, stream);
}

// Box-Muller pairs: the plain kernel when vectors start at even draws, else the pair tile
// kernel (tunable "pair_lds"; the plain kernel then takes the pair after the wave itself).
template <class Op, class T>
tk_status run_pairs(Op op, T *out, uint64_t start, uint64_t n, hipStream_t stream) {
  set_geometry(op, out, start, n);
  if (((op.start + op.head) & 1u) == 0 || !config().pair_lds) return launch_vec(op, stream);
  return launch_pair_tile(op, stream);
}

// Philox fills whose vectors straddle blocks when (start + head) & mask != 0: the tile
// kernel or the overlapping-wave kernel then (tunable "philox_lds"), the plain one
// otherwise.
template <class Op, class T>
tk_status run_straddling(Op op, T *out, uint64_t start, uint64_t n, uint32_t mask, hipStream_t stream) {
  set_geometry(op, out, start, n);
  if (((op.start + op.head) & mask) == 0) return launch_vec(op, stream);
  return config().philox_lds ? launch_philox_tile(op, stream) : launch_vec_overlap(op, stream);
}

// The same for ops without a tile form (the Philox Box-Muller pairs).
template <class Op, class T>
tk_status run_straddling_overlap(Op op, T *out, uint64_t start, uint64_t n, uint32_t mask, hipStream_t stream) {
  set_geometry(op, out, start, n);
  return ((op.start + op.head) & mask) ? launch_vec_overlap(op, stream) : launch_vec(op, stream);
}

static Below32Params below32_params(uint32_t key, uint32_t bound, int64_t low) {
  Below32Params p;
  p.hk = host_lowbias32(key);
  p.hkp = host_substream_key(key, kPurposeBelow32);
  p.s = bound;
  p.t = (uint32_t)(0u - bound) % bound;
  p.low = low;
  return p;
}

template <class T>
static tk_status below64(uint32_t key, uint64_t start_draw, uint64_t n, int64_t low, uint64_t bound, T *out,
                         hipStream_t stream) {
  const uint32_t hk = host_lowbias32(key), hkp = host_substream_key(key, kPurposeBelow64);
  const uint64_t t = (0ull - bound) % bound;
  if (bound <= 0xFFFFFFFFull) {
    OpBelow64<T, true> op{};
    op.hk = hk; op.hkp = hkp; op.s = bound; op.t = t; op.low = low;
    return run_simple(op, out, start_draw, n, stream);
  }
  OpBelow64<T, false> op{};
  op.hk = hk; op.hkp = hkp; op.s = bound; op.t = t; op.low = low;
  return run_simple(op, out, start_draw, n, stream);
}

}  // namespace

extern "C" {

tk_status tk_fill_constant_u32(uint32_t value, uint64_t n, uint32_t *out, hipStream_t stream) {
  if (n == 0) return TK_OK;
  if (!out || !elem_aligned(out)) return TK_EINVAL;
  if (n > (~0ull >> 2)) return TK_ERANGE;  // n * 4 bytes must be addressable
  OpConst op{};
  op.value = value;
  op.work = (uint32_t)config().const_work;
  return run_simple(op, out, 0, n, stream);
}

tk_status tk_fill_u32(uint32_t key, uint64_t start_draw, uint64_t n, uint32_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW32);
  OpWord32<false> op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW32);
  OpWord32<true> op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, (uint32_t *)out, start_draw, n, stream);
}

tk_status tk_fill_u64(uint32_t key, uint64_t start_draw, uint64_t n, uint64_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW64);
  OpWord64<false> op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW64);
  OpWord64<true> op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, (uint64_t *)out, start_draw, n, stream);
}

tk_status tk_fill_u16(uint32_t key, uint64_t start_draw, uint64_t n, uint16_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxU16);
  OpSub16<false> op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_f16_bits(uint32_t key, uint64_t start_draw, uint64_t n, uint16_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxU16);
  OpSub16<true> op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_u8(uint32_t key, uint64_t start_draw, uint64_t n, uint8_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxU8);
  OpU8 op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_bool(uint32_t key, uint64_t start_draw, uint64_t n, uint8_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxBool);
  OpBool op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_u32_below(uint32_t key, uint64_t start_draw, uint64_t n, uint32_t bound, uint32_t *out,
                            hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  TK_PRECHECK(out, kMaxW32);
  OpBelow32<uint32_t> op{};
  op.p = below32_params(key, bound, 0);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_i32_below(uint32_t key, uint64_t start_draw, uint64_t n, int32_t low, uint32_t bound,
                            int32_t *out, hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  if ((int64_t)low + (int64_t)bound - 1 > (int64_t)INT32_MAX) return TK_ERANGE;
  TK_PRECHECK(out, kMaxW32);
  OpBelow32<int32_t> op{};
  op.p = below32_params(key, bound, low);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_i64_below32(uint32_t key, uint64_t start_draw, uint64_t n, int64_t low, uint32_t bound,
                              int64_t *out, hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  if ((__int128)low + (__int128)bound - 1 > (__int128)INT64_MAX) return TK_ERANGE;
  TK_PRECHECK(out, kMaxW32);
  OpBelow32To64 op{};
  op.p = below32_params(key, bound, low);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_u64_below(uint32_t key, uint64_t start_draw, uint64_t n, uint64_t bound, uint64_t *out,
                            hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  TK_PRECHECK(out, kMaxW64);
  return below64<uint64_t>(key, start_draw, n, 0, bound, out, stream);
}

tk_status tk_fill_i64_below(uint32_t key, uint64_t start_draw, uint64_t n, int64_t low, uint64_t bound,
                            int64_t *out, hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  if ((__int128)low + (__int128)bound - 1 > (__int128)INT64_MAX) return TK_ERANGE;
  TK_PRECHECK(out, kMaxW64);
  return below64<int64_t>(key, start_draw, n, low, bound, out, stream);
}

tk_status tk_fill_normal_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW32);
  OpNormalF32<false> op{};
  op.hk = host_lowbias32(key);
  return run_pairs(op, out, start_draw, n, stream);
}

tk_status tk_fill_normal_f32_half_turn(uint32_t key, uint64_t start_draw, uint64_t n, float *out,
                                       hipStream_t stream) {
  TK_PRECHECK(out, kMaxW32);
  OpNormalF32<true> op{};
  op.hk = host_lowbias32(key);
  return run_pairs(op, out, start_draw, n, stream);
}

tk_status tk_fill_randn_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW64);  // counter c reads words 2c and 2c + 1
  OpRandnF32 op{};
  op.hk = host_lowbias32(key);
  return run_simple(op, out, start_draw, n, stream);
}

tk_status tk_fill_exponential_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW64);
  OpExpF64 op{};
  op.hk = host_lowbias32(key);
  return run_exp(op, (uint64_t *)out, start_draw, n, stream);
}

tk_status tk_fill_exponential_f32(uint32_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxW32);
  OpExpF32 op{};
  op.hk = host_lowbias32(key);
  return run_exp(op, (uint32_t *)out, start_draw, n, stream);
}

tk_status tk_dropout_f32(uint32_t key, uint64_t start_draw, uint64_t n, float p, const float *x, float *y,
                         uint8_t *mask, hipStream_t stream) {
  if (!(p >= 0.0f && p < 1.0f)) return TK_EINVAL;
  if (n == 0) return TK_OK;
  if (!x || !y || !elem_aligned(x) || !elem_aligned(y)) return TK_EINVAL;
  if (x != y) {  // in place is allowed; any other overlap is not
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y, bytes = (uintptr_t)(n * sizeof(float));
    if (xa < ya + bytes && ya < xa + bytes) return TK_EINVAL;
  }
  tk_status st = check_draws(start_draw, n, kMaxW32);
  if (st != TK_OK) return st;
  OpDropout op{};
  set_geometry(op, y, start_draw, n);
  op.x = x;
  op.mask = mask;
  op.hk = host_lowbias32(key);
  op.p = p;
  op.q = 1.0f - p;
  op.x_vec = (((uintptr_t)(x + op.head)) & 15u) == 0;
  op.mask_word = mask && (((uintptr_t)(mask + op.head)) & 3u) == 0;
  return launch_vec_nt(op, stream);
}

tk_status tk_dropout_backward_f32(uint32_t key, uint64_t start_draw, uint64_t n, float p, const float *dy,
                                  float *dx, hipStream_t stream) {
  return tk_dropout_f32(key, start_draw, n, p, dy, dx, nullptr, stream);
}

tk_status tk_philox_fill_u32(uint64_t key, uint64_t start_draw, uint64_t n, uint32_t *out, hipStream_t stream) {
  TK_PRECHECK(out, ~0ull);
  OpPhilox32<false> op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32);
  return run_straddling(op, out, start_draw, n, 3u, stream);
}

tk_status tk_philox_fill_f32(uint64_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream) {
  TK_PRECHECK(out, ~0ull);
  OpPhilox32<true> op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32);
  return run_straddling(op, (uint32_t *)out, start_draw, n, 3u, stream);
}

tk_status tk_philox_fill_u64(uint64_t key, uint64_t start_draw, uint64_t n, uint64_t *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxPhilox64);
  OpPhilox64<false> op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32);
  return run_straddling(op, out, start_draw, n, 1u, stream);
}

tk_status tk_philox_fill_u32_below(uint64_t key, uint64_t start_draw, uint64_t n, uint32_t bound, uint32_t *out,
                                   hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  TK_PRECHECK(out, ~0ull);
  OpPhiloxBelow32 op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32);
  op.s = bound;
  op.t = (uint32_t)(0u - bound) % bound;
  return run_straddling(op, out, start_draw, n, 3u, stream);
}

tk_status tk_philox_fill_u64_below(uint64_t key, uint64_t start_draw, uint64_t n, uint64_t bound, uint64_t *out,
                                   hipStream_t stream) {
  if (bound == 0) return TK_EINVAL;
  TK_PRECHECK(out, kMaxPhilox64);
  const uint64_t t = (0ull - bound) % bound;
  if (bound <= 0xFFFFFFFFull) {
    OpPhiloxBelow64<true> op{};
    op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32); op.s = bound; op.t = t;
    return run_straddling(op, out, start_draw, n, 1u, stream);
  }
  OpPhiloxBelow64<false> op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32); op.s = bound; op.t = t;
  return run_straddling(op, out, start_draw, n, 1u, stream);
}

tk_status tk_philox_fill_normal_f32(uint64_t key, uint64_t start_draw, uint64_t n, float *out, hipStream_t stream) {
  TK_PRECHECK(out, ~0ull);
  OpPhiloxNormalF32 op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32);
  return run_straddling_overlap(op, out, start_draw, n, 3u, stream);
}

tk_status tk_philox_fill_f64(uint64_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  TK_PRECHECK(out, kMaxPhilox64);
  OpPhilox64<true> op{};
  op.k0 = (uint32_t)key; op.k1 = (uint32_t)(key >> 32);
  return run_straddling(op, (uint64_t *)out, start_draw, n, 1u, stream);
}

}  // extern "C"
