// tk_ziggurat.hip -- f64 normal fill: the 1024-layer ziggurat.
//
// tandem-sycl, "Design", §Normals: element i takes 64-bit draw i; about 0.43 % of draws
// miss the fast path and continue on the per-index substream split(i) of
// sub(key, PURPOSE_NORMAL64).
//
// Default (fused) path, one kernel.  Each work-group copies the 16 KiB layer table (pairs
// {X[L] 2^-53, X[L+1]}) to LDS, writes four tiles of fast-path values with 16-byte stores
// (two elements per lane), and queues its misses in LDS through wave ballots, one region
// per wave, without atomics.  After a barrier it finishes its own ~9 misses (the wedge
// test against exp(-x^2/2), or the tail beyond r) and rewrites them while their lines are
// still in L2.  A group whose queue overflows walks its own elements again, so the result
// never depends on the queue sizes.
//
// Two-kernel path (TK_ZIG_MODE=split, or tk_debug_set_normal_f64_mode(1)), the pages'
// shape: the table pass writes each group's queue to the group's own slot of a device
// miss list, and entries beyond the slot to an overflow list with one atomic each; the
// continuation pass compacts the slots and finishes the misses, one per lane, and walks
// the whole fill if the overflow list itself overflowed.  Both paths give the same values.
//
// The table is never read through scalar/constant memory: divergent layer reads would
// serialize there (the page measured a drop to 27 GiB/s that way).  The table is constant
// per-device state.  The lists and the counters are per-device state shared by all
// streams: fills that use them (the two-kernel path, and fills counted for the miss-count
// test hook) wait on the previous such fill's event.  The default fused fill uses none of
// them and needs no event.  The pages append each group's misses with one
// atomic add; at ~130 thousand groups per 2^28-element fill that would serialize on one
// address, hence the per-group slots.
#include <math.h>

#include <mutex>
#include <vector>

#include "tk_device.h"
#include "tk_internal.h"
#include "zig1024.inc"

namespace tk {

constexpr uint32_t kSlotPerTile = 16;  // miss entries a work-group keeps per 4 KiB tile

// Miss-queue entries per wave of a table-pass group of kB lanes and T tiles: 4 per tile
// of 512 elements (2.2 expected misses per 256-lane tile, so 16 per 256-lane tile), and at
// least 8 (a wave sees Poisson(0.55) misses per tile; more than 8 happens about once in
// 1e8 waves, and then the group walks its elements again).
constexpr uint32_t zig_wave_entries(int T) { return 4u * (uint32_t)T > 8u ? 4u * (uint32_t)T : 8u; }
constexpr uint32_t zig_slot_entries(int kB, int T) { return (uint32_t)(kB / 64) * zig_wave_entries(T); }

struct ZigArgs {
  double *out;
  uint64_t start;  // draw of element 0
  uint64_t n;
  uint64_t head;   // 0 or 1 element before the first 16-byte boundary
  uint64_t nvec;   // whole 16-byte vectors (two elements each)
  uint32_t tail;   // 0 or 1 element after them
  uint32_t hk;     // lowbias32 source: lowbias32(key)
  uint32_t hkp;    //   and lowbias32(sub(key, NORM))
  uint32_t k0, k1; // Philox source: the key
  const double2 *xx;  // {X[L] * 2^-53, X[L+1]}, L < 1024
  const double *f;    // F[0 .. 1024]
  double r;
  uint32_t ngroups;    // table-pass work-groups = slots
  uint32_t slot_size;  // entries reserved per slot
  uint32_t slot_cap;   // entries used per slot (<= slot_size)
  uint32_t *counts;    // [ngroups] misses kept in each slot (fused: seen; null when not counted)
  uint32_t *slots;     // [ngroups * slot_size]
  uint32_t *ovf;       // overflow list
  uint32_t ovf_cap;
  uint32_t *ctr;   // [0] overflow entries (cleared before each fill)
};

// The fast path of a draw (lo, hi): layer L = lo & 1023, sign bit 10, m = d >> 11 the
// top 53 bits; x = m * (X[L] 2^-53) equals u * X[L] with u = m 2^-53 bit for bit
// (scaling by a power of two is exact), and the draw is accepted when x < X[L+1].
// m is assembled exactly: hi 2^21 + (lo >> 11) < 2^53 in one fused operation.
__device__ __forceinline__ double zig_x(uint32_t lo, uint32_t hi, double scaled_edge) {
  const double m = __builtin_fma((double)hi, 0x1p21, (double)(lo >> 11));
  return m * scaled_edge;
}

__device__ __forceinline__ bool zig_fast(const double2 *tab, uint32_t lo, uint32_t hi, double *val) {
  const double2 e = tab[lo & 1023u];
  const double x = zig_x(lo, hi, e.x);
  // the sign is bit 10 of the draw, moved to bit 63 (x >= 0, so this is -x when set):
  // x_hi ^ ((lo << 21) & 0x80000000) as one v_bitop3 (truth table 0x78 = a ^ (b & c))
  const uint64_t xb = (uint64_t)__double_as_longlong(x);
  const uint32_t sh = __builtin_amdgcn_bitop3_b32((uint32_t)(xb >> 32), lo << 21, 0x80000000u, 0x78);
  *val = __longlong_as_double((long long)(((uint64_t)sh << 32) | (uint32_t)xb));
  return x < e.y;
}

// The four words of vector v: counters c0 .. c0+3 with c0 = 2 (start + head + 2v).  When
// start + head is even, c0 is a multiple of 4 and (c0 + j) ^ hk = c0 ^ (hk ^ j), one xor
// with a uniform value per word.  Philox: the lane's block, or at odd start + head its
// second half and the next lane's first (every lane of the wave must call this).
template <bool kAligned4, bool kPhilox>
__device__ __forceinline__ void zig_words(const ZigArgs &a, uint64_t v, uint32_t w[4]) {
  if (kPhilox) {
    const uint4 b = philox_words(2 * (a.start + a.head + 2 * v), a.k0, a.k1);
    w[0] = b.x; w[1] = b.y; w[2] = b.z; w[3] = b.w;
    return;
  }
  const uint32_t c0 = 2u * (uint32_t)(a.start + a.head + 2 * v);
  if (kAligned4) {
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) w[j] = lowbias32(c0 ^ (a.hk ^ j));
  } else {
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) w[j] = word(a.hk, c0 + j);
  }
}

// The primary 64-bit draw of element k: words 2i (lo) and 2i+1 (hi), i = start + k.
template <bool kPhilox>
__device__ __forceinline__ void zig_primary(const ZigArgs &a, uint64_t k, uint32_t *lo, uint32_t *hi) {
  if (kPhilox) {
    const uint64_t w = 2 * (a.start + k);
    *lo = philox_word(w, a.k0, a.k1);
    *hi = philox_word(w + 1, a.k0, a.k1);
  } else {
    const uint32_t c = 2u * (uint32_t)(a.start + k);
    *lo = word(a.hk, c);
    *hi = word(a.hk, c + 1);
  }
}

// The work-group's miss queue is one region per wave, so a wave appends without atomics:
// it counts its misses in a wave-uniform register and ranks them with ballots.  `q` is
// the wave's region, `cap` its usable entries.  Past `cap`, a fused table pass only
// counts the miss (the group re-walks); the two-kernel pass appends it to the overflow
// list.
struct WaveQueue {
  uint32_t *q;
  uint32_t cap;
  uint32_t n;  // misses seen (wave-uniform)
};

template <bool kFused>
__device__ __forceinline__ void queue_put(uint32_t slot, uint32_t k, const WaveQueue &wq, const ZigArgs &a) {
  if (slot < wq.cap) {
    wq.q[slot] = k;
  } else if (!kFused) {
    const uint32_t g = atomicAdd(&a.ctr[0], 1u);
    if (g < a.ovf_cap) a.ovf[g] = k;
  }
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Appends the lane's misses (element k0 when p0, k0 + 1 when p1) to the wave's region:
// two ballots, ranks from mbcnt.  Called by all lanes of the wave.
template <bool kFused>
__device__ __forceinline__ void enqueue2(bool p0, bool p1, uint32_t k0, WaveQueue &wq, const ZigArgs &a) {
  const uint64_t m0 = __builtin_amdgcn_ballot_w64(p0), m1 = __builtin_amdgcn_ballot_w64(p1);
  if ((m0 | m1) == 0) return;
  const uint32_t c0 = (uint32_t)__popcll(m0);
  if (p0) queue_put<kFused>(wq.n + lane_rank(m0), k0, wq, a);
  if (p1) queue_put<kFused>(wq.n + c0 + lane_rank(m1), k0 + 1, wq, a);
  wq.n += c0 + (uint32_t)__popcll(m1);
}

template <bool kPhilox>
__device__ double zig_slow(const ZigArgs &a, uint64_t k);

// One tile: 256 lanes, two elements each, from the lane's four words.  kCheck guards
// vectors past the end (only the last group needs it).
template <bool kCheck, bool kFused, bool kNT>
__device__ __forceinline__ void zig_tile(const ZigArgs &a, const double2 *tab, uint64_t v, const uint32_t w[4],
                                         WaveQueue &wq) {
  const bool in = !kCheck || v < a.nvec;
  double y0, y1;
  const bool f0 = zig_fast(tab, w[0], w[1], &y0);
  const bool f1 = zig_fast(tab, w[2], w[3], &y1);
  if (in) {
    uint4 o;
    o.x = (uint32_t)__double_as_longlong(y0);
    o.y = (uint32_t)((uint64_t)__double_as_longlong(y0) >> 32);
    o.z = (uint32_t)__double_as_longlong(y1);
    o.w = (uint32_t)((uint64_t)__double_as_longlong(y1) >> 32);
    store16<kNT>(a.out + a.head + 2 * v, o);
  }
  enqueue2<kFused>(in && !f0, in && !f1, (uint32_t)(a.head + 2 * v), wq, a);
}

// The group's T tiles.  Every lane's words for all of them are hashed first, while the
// copy of the layer table to LDS (kLds) is still in flight: the loads are issued, the hashes
// run, and only then does the lane wait for the loads, write LDS and meet the barrier.
template <int kB, int T, bool kLds, bool kAligned4, bool kFused, bool kNT, bool kPhilox>
__device__ __forceinline__ void zig_tiles(const ZigArgs &a, double2 *lds_tab, WaveQueue &wq) {
  const uint64_t v0 = (uint64_t)blockIdx.x * T * kB + threadIdx.x;
  uint32_t w[T][4];
  if (kLds) {
    constexpr int kPer = 1024 / kB;
    double2 t[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) t[r] = a.xx[threadIdx.x + r * kB];
#pragma unroll
    for (int i = 0; i < T; ++i) zig_words<kAligned4, kPhilox>(a, v0 + (uint64_t)i * kB, w[i]);
#pragma unroll
    for (int r = 0; r < kPer; ++r) lds_tab[threadIdx.x + r * kB] = t[r];
    __syncthreads();
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) zig_words<kAligned4, kPhilox>(a, v0 + (uint64_t)i * kB, w[i]);
  }
  const double2 *tab = kLds ? lds_tab : a.xx;
  if ((uint64_t)(blockIdx.x + 1) * T * kB <= a.nvec) {
#pragma unroll
    for (int i = 0; i < T; ++i) zig_tile<false, kFused, kNT>(a, tab, v0 + (uint64_t)i * kB, w[i], wq);
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) zig_tile<true, kFused, kNT>(a, tab, v0 + (uint64_t)i * kB, w[i], wq);
  }
}

// Table pass: T consecutive tiles of kB lanes (one 16-byte vector per lane each) per
// work-group.  With kLds the 16 KiB layer table is first copied to LDS (one copy per T
// tiles) and gathered from there; otherwise the gathers go to the table in device memory
// through L1/L2.  Misses go to the queue region of their wave (zig_wave_entries(T)
// entries; a wave expects 0.55 misses per tile), appended without atomics.
// With kFused the work-group finishes its own misses after its stores, while the lines it
// just wrote are still in L2; a group with a wave that found more misses than its region
// holds (probability ~1e-10 per wave) walks its own elements again and finishes every miss
// it meets, so nothing leaves the work-group.  Otherwise the queue goes to the group's
// slot for the continuation pass.
template <int kB, int T, bool kLds, bool kNT, bool kFused, bool kPhilox>
__global__ __launch_bounds__(kB) void k_zig_table_pass(ZigArgs a) {
  constexpr uint32_t kWaves = kB / 64;
  constexpr uint32_t kPerWave = zig_wave_entries(T);  // a wave's share of the group's slot
  constexpr uint32_t kRegion = kPerWave + (kFused ? 1u : 0u);  // fused: + an edge element (waves 0 and 1)
  __shared__ double2 lds_tab[kLds ? 1024 : 1];
  __shared__ uint32_t q[kWaves * kRegion];
  __shared__ uint32_t wave_n[kWaves];
  const uint32_t w = threadIdx.x >> 6;
  // entries a wave keeps: its share of the group's slot capacity (smaller when a test
  // shrinks the slots), plus the edge element in the fused pass
  const uint32_t share = (a.slot_cap + kWaves - 1) / kWaves;
  WaveQueue wq{q + w * kRegion, (share < kPerWave ? share : kPerWave) + (kFused ? 1u : 0u), 0u};
  // (start + head) & 1 is the same for the whole grid: every thread meets the barrier in
  // zig_tiles on the same branch
  if (((a.start + a.head) & 1u) == 0) zig_tiles<kB, T, kLds, true, kFused, kNT, kPhilox>(a, lds_tab, wq);
  else zig_tiles<kB, T, kLds, false, kFused, kNT, kPhilox>(a, lds_tab, wq);
  const double2 *tab = kLds ? lds_tab : a.xx;
  if (blockIdx.x == 0) {  // the element before the first boundary and the one after the last vector
    const uint32_t t = threadIdx.x;
    bool edge = false;
    uint64_t k = 0;
    if (t == 0 && a.head) { edge = true; k = 0; }
    if (t == 64 && a.tail) { edge = true; k = a.head + 2 * a.nvec; }
    bool fast = true;
    if (edge) {
      uint32_t lo, hi;
      zig_primary<kPhilox>(a, k, &lo, &hi);
      double y;
      fast = zig_fast(tab, lo, hi, &y);
      a.out[k] = y;
    }
    enqueue2<kFused>(edge && !fast, false, (uint32_t)k, wq, a);
  }
  if (lane_id() == 0) wave_n[w] = wq.n;
  __syncthreads();
  // the kept entries of all regions, numbered in wave order
  uint32_t seen = 0, kept = 0, off[kWaves];
  bool over = false;
#pragma unroll
  for (uint32_t i = 0; i < kWaves; ++i) {
    const uint32_t ni = wave_n[i];
    seen += ni;
    over |= ni > wq.cap;
    off[i] = kept;
    kept += ni < wq.cap ? ni : wq.cap;
  }
  auto entry = [&](uint32_t j) {  // j < kept
    uint32_t i = 0;
#pragma unroll
    for (uint32_t r = 1; r < kWaves; ++r) i += j >= off[r] ? 1u : 0u;
    return q[i * kRegion + (j - off[i])];
  };
  if (kFused) {
    if (threadIdx.x == 0 && a.counts) a.counts[blockIdx.x] = seen;
    if (!over) {
      // Each value here replaces the placeholder a wave of this group stored in its tile
      // before the barrier.  The barrier does not wait for those stores to complete; the
      // order comes from the group running on one CU (no tgsplit), whose waves' vector
      // memory instructions pass through one texture path and L1 in issue order to the L2
      // channel that owns the address, so this later store lands after the placeholder.
      for (uint32_t j = threadIdx.x; j < kept; j += kB) {
        const uint32_t k = entry(j);
        a.out[k] = zig_slow<kPhilox>(a, k);
      }
    } else {  // a wave had more misses than its region holds: walk the group's elements again
      const uint64_t e0 = a.head + (uint64_t)blockIdx.x * T * kB * 2;
      uint64_t e1 = e0 + (uint64_t)T * kB * 2;
      if (e1 > a.head + 2 * a.nvec) e1 = a.head + 2 * a.nvec;
      for (uint64_t k = e0 + threadIdx.x; k < e1; k += kB) {
        uint32_t lo, hi;
        zig_primary<kPhilox>(a, k, &lo, &hi);
        double y;
        if (!zig_fast(a.xx, lo, hi, &y)) a.out[k] = zig_slow<kPhilox>(a, k);
      }
      if (blockIdx.x == 0 && threadIdx.x < 2) {  // and the edge elements
        const bool has = threadIdx.x == 0 ? a.head != 0 : a.tail != 0;
        const uint64_t k = threadIdx.x == 0 ? 0 : a.head + 2 * a.nvec;
        if (has) {
          uint32_t lo, hi;
          zig_primary<kPhilox>(a, k, &lo, &hi);
          double y;
          if (!zig_fast(a.xx, lo, hi, &y)) a.out[k] = zig_slow<kPhilox>(a, k);
        }
      }
    }
  } else {  // the kept entries go to the group's slot (at most kWaves * kPerWave = slot_size)
    if (threadIdx.x == 0) a.counts[blockIdx.x] = kept;
    for (uint32_t j = threadIdx.x; j < kept; j += kB) a.slots[(uint64_t)blockIdx.x * a.slot_size + j] = entry(j);
  }
}

// Finishes a draw (lo, hi) that left the fast path: wedge, tail and restarts read the
// substream `ss` in order (split(i) of sub(key, NORM) for lowbias32, the NORM Philox
// substream of draw i for Philox).
template <class Sub>
__device__ double zig_finish(const ZigArgs &a, uint32_t lo, uint32_t hi, Sub ss) {
  const uint32_t cap_words = 2u * kSubstreamCap;
  for (;;) {
    const uint32_t L = lo & 1023u;
    const bool neg = (lo & 1024u) != 0;
    const double2 e = a.xx[L];
    const double x = zig_x(lo, hi, e.x);
    if (x < e.y) return neg ? -x : x;
    if (L == 0) {  // tail beyond r (Marsaglia & Tsang)
      for (;;) {
        if (ss.pos + 4u > cap_words) return NAN;
        const uint64_t da = ss.next64(), db = ss.next64();
        const double ua = (double)((da >> 11) + 1u) * 0x1p-53;
        const double ub = (double)((db >> 11) + 1u) * 0x1p-53;
        const double xi = -log(ua) / a.r;
        const double eta = -log(ub);
        if (eta + eta > xi * xi) {
          const double t = a.r + xi;
          return neg ? -t : t;
        }
      }
    }
    if (ss.pos + 2u > cap_words) return NAN;
    const double y = (double)(ss.next64() >> 11) * 0x1p-53;
    const double fl = a.f[L], fh = a.f[L + 1];
    if (fl + y * (fh - fl) < exp(-0.5 * (x * x))) return neg ? -x : x;
    if (ss.pos + 2u > cap_words) return NAN;
    const uint64_t d = ss.next64();
    lo = (uint32_t)d;
    hi = (uint32_t)(d >> 32);
  }
}

// Finishes element k from its primary draw.
template <bool kPhilox>
__device__ double zig_slow(const ZigArgs &a, uint64_t k) {
  uint32_t lo, hi;
  zig_primary<kPhilox>(a, k, &lo, &hi);
  if (kPhilox) return zig_finish(a, lo, hi, PhiloxSub(a.k0, a.k1, a.start + k, kPurposeNormal64));
  return zig_finish(a, lo, hi, Substream(a.hkp, (uint32_t)(a.start + k)));
}

// Exclusive prefix sum of v over the work-group; *total receives the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wave_sums, uint32_t *total) {
  const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_sums[w] = x;
  __syncthreads();
  uint32_t base = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) {
    if (i < w) base += wave_sums[i];
    sum += wave_sums[i];
  }
  *total = sum;
  return base + x - v;
}

// Continuation pass.  Block b compacts the misses of table-pass groups
// [b * gpb, (b + 1) * gpb) (gpb chosen so a block sees about 256 groups' worth of tiles)
// and spreads them over its lanes, so every lane finishes about two misses.
template <bool kPhilox>
__global__ __launch_bounds__(kBlock) void k_zig_continue(ZigArgs a, uint32_t gpb) {
  __shared__ uint32_t s_ovf;
  __shared__ uint32_t offs[kBlock + 1];
  __shared__ uint32_t wave_sums[kBlock / 64];
  if (threadIdx.x == 0) s_ovf = __hip_atomic_load(&a.ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t ovf = s_ovf;
  if (ovf <= a.ovf_cap) {
    const uint64_t g0 = (uint64_t)blockIdx.x * gpb;
    const uint64_t g = g0 + threadIdx.x;
    const uint32_t cnt = (threadIdx.x < gpb && g < a.ngroups) ? a.counts[g] : 0u;
    uint32_t total;
    const uint32_t off = block_exclusive_scan(cnt, wave_sums, &total);
    if (threadIdx.x < gpb) offs[threadIdx.x] = off;
    if (threadIdx.x == 0) offs[gpb] = total;
    __syncthreads();
    for (uint32_t m = threadIdx.x; m < total; m += kBlock) {
      uint32_t lo = 0, hi = gpb;  // the group j with offs[j] <= m < offs[j + 1]
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (offs[mid] <= m) lo = mid;
        else hi = mid;
      }
      const uint32_t k = a.slots[(g0 + lo) * a.slot_size + (m - offs[lo])];
      a.out[k] = zig_slow<kPhilox>(a, k);
    }
    const uint64_t gid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    for (uint64_t j = gid; j < ovf; j += (uint64_t)gridDim.x * kBlock) {
      const uint32_t k = a.ovf[j];
      a.out[k] = zig_slow<kPhilox>(a, k);
    }
  } else {  // the overflow list overflowed: find the misses by walking the whole fill
    const uint64_t stride = (uint64_t)gridDim.x * kBlock;
    for (uint64_t k = (uint64_t)blockIdx.x * kBlock + threadIdx.x; k < a.n; k += stride) {
      uint32_t lo, hi;
      zig_primary<kPhilox>(a, k, &lo, &hi);
      double y;
      if (!zig_fast(a.xx, lo, hi, &y)) a.out[k] = zig_slow<kPhilox>(a, k);
    }
  }
}

// Clears the overflow count before a fill.  A kernel rather than a
// memset, and no end-of-pass "last block resets" scheme: that needs a device-scope
// release fence per block, which on MI355X writes back the whole L2 (full of the table
// pass's output) once per block.
__global__ void k_zig_reset(uint32_t *ctr) {
  if (threadIdx.x == 0) ctr[0] = 0u;
}

// ---------------------------------------------------------------------------------------
// Per-device state
// ---------------------------------------------------------------------------------------
struct ZigDevice {
  std::mutex m;
  bool ready = false;
  double2 *xx = nullptr;
  double *f = nullptr;
  uint32_t *ctr = nullptr;
  uint32_t *counts = nullptr;
  uint32_t *slots = nullptr;
  uint64_t groups_cap = 0;    // counts allocated
  uint64_t slot_words = 0;    // slot entries allocated
  uint32_t *ovf = nullptr;
  uint64_t ovf_alloc = 0;
  uint64_t last_groups = 0;   // table-pass groups of the last counted fill
  bool last_fused = false;
  bool last_counted = false;  // the last fill on this device kept its miss counts
  hipEvent_t last = nullptr;
  bool recorded = false;
};

static ZigDevice g_zig[kMaxDevices];
static std::mutex g_cap_mutex;
static uint32_t g_debug_slot_cap = 0;
static int g_debug_mode = 0;  // 0: configured default, 1: two kernels, 2: fused
static uint64_t g_debug_ovf_cap = 0;
constexpr uint64_t kOvfDefault = 65536;

// Releases the constant tables, the counter and the event (a failed first fill).
static void zig_release(ZigDevice &d) {
  (void)device_free(d.xx, TK_ZIG_LAYERS * sizeof(double2));
  (void)device_free(d.f, sizeof(tk_zig_f));
  (void)device_free(d.ctr, 4 * sizeof(uint32_t));
  d.xx = nullptr;
  d.f = nullptr;
  d.ctr = nullptr;
  if (d.last) (void)hipEventDestroy(d.last);
  d.last = nullptr;
}

static tk_status zig_create(ZigDevice &d) {
  double2 pairs[TK_ZIG_LAYERS];
  for (int L = 0; L < TK_ZIG_LAYERS; ++L) pairs[L] = make_double2(tk_zig_x[L] * 0x1p-53, tk_zig_x[L + 1]);
  if (device_alloc((void **)&d.xx, sizeof(pairs)) != hipSuccess) return TK_ENOMEM;
  if (device_alloc((void **)&d.f, sizeof(tk_zig_f)) != hipSuccess) return TK_ENOMEM;
  if (device_alloc((void **)&d.ctr, 4 * sizeof(uint32_t)) != hipSuccess) return TK_ENOMEM;
  tk_status st;
  if ((st = hip_status(hipMemcpy(d.xx, pairs, sizeof(pairs), hipMemcpyHostToDevice))) != TK_OK) return st;
  if ((st = hip_status(hipMemcpy(d.f, tk_zig_f, sizeof(tk_zig_f), hipMemcpyHostToDevice))) != TK_OK) return st;
  if ((st = hip_status(hipMemset(d.ctr, 0, 4 * sizeof(uint32_t)))) != TK_OK) return st;
  return hip_status(hipEventCreateWithFlags(&d.last, hipEventDisableTiming));
}

// The device's state on its first fill; a failure releases whatever was created, so the
// next fill starts again from nothing.
static tk_status zig_init(ZigDevice &d) {
  if (d.ready) return TK_OK;
  const tk_status st = zig_create(d);
  if (st != TK_OK)
    zig_release(d);
  else
    d.ready = true;
  return st;
}

// Releases the miss counts, the slot arrays and the overflow list; the last fill's miss
// count goes with them.
static void zig_release_lists(ZigDevice &d) {
  (void)device_free(d.counts, d.groups_cap * sizeof(uint32_t));
  (void)device_free(d.slots, d.slot_words * sizeof(uint32_t));
  (void)device_free(d.ovf, d.ovf_alloc * sizeof(uint32_t));
  d.counts = d.slots = d.ovf = nullptr;
  d.groups_cap = d.slot_words = d.ovf_alloc = 0;
  d.last_counted = false;
}

// Grows the miss counts, the slot arrays and the overflow list; the previous fill may
// still read them, so it is waited for first.  If an allocation fails, all three are
// released (the next fill allocates them again).
static tk_status zig_reserve(ZigDevice &d, uint64_t groups, uint64_t slot_words, uint64_t ovf_cap) {
  if (groups <= d.groups_cap && slot_words <= d.slot_words && ovf_cap <= d.ovf_alloc) return TK_OK;
  tk_status st;
  if (d.recorded && (st = hip_status(hipEventSynchronize(d.last))) != TK_OK) return st;
  st = TK_OK;
  if (groups > d.groups_cap) {
    (void)device_free(d.counts, d.groups_cap * sizeof(uint32_t));
    d.counts = nullptr;
    d.groups_cap = 0;
    if (device_alloc((void **)&d.counts, groups * sizeof(uint32_t)) == hipSuccess)
      d.groups_cap = groups;
    else
      st = TK_ENOMEM;
  }
  if (st == TK_OK && slot_words > d.slot_words) {
    (void)device_free(d.slots, d.slot_words * sizeof(uint32_t));
    d.slots = nullptr;
    d.slot_words = 0;
    if (device_alloc((void **)&d.slots, slot_words * sizeof(uint32_t)) == hipSuccess)
      d.slot_words = slot_words;
    else
      st = TK_ENOMEM;
  }
  if (st == TK_OK && ovf_cap > d.ovf_alloc) {
    (void)device_free(d.ovf, d.ovf_alloc * sizeof(uint32_t));
    d.ovf = nullptr;
    d.ovf_alloc = 0;
    if (device_alloc((void **)&d.ovf, ovf_cap * sizeof(uint32_t)) == hipSuccess)
      d.ovf_alloc = ovf_cap;
    else
      st = TK_ENOMEM;
  }
  if (st != TK_OK) zig_release_lists(d);
  return st;
}

template <int kB, int T, bool kLds, bool kFused, bool kPhilox>
static void launch_table_pass(const ZigArgs &a, hipStream_t stream) {
  if (config().nt_stores)
    hipLaunchKernelGGL((k_zig_table_pass<kB, T, kLds, true, kFused, kPhilox>), dim3(a.ngroups), dim3(kB),
                       (uint32_t)config().zig_lds_pad, stream, a);
  else
    hipLaunchKernelGGL((k_zig_table_pass<kB, T, kLds, false, kFused, kPhilox>), dim3(a.ngroups), dim3(kB),
                       (uint32_t)config().zig_lds_pad, stream,
                       a);
}

// The table-pass shapes that are built: 256-lane groups with 2 .. 16 tiles (LDS or global
// table), or one tile gathering from the global table.  (1024-lane groups measured slower
// at every tile count: their 16-wave slots wait for the one wave that finishes the misses.)
struct ZigShape {
  int block, tiles;
  bool lds;
};

static ZigShape zig_shape() {
  const int zt = config().zig_tiles;
  ZigShape sh;
  sh.block = kBlock;
  sh.tiles = zt >= 16 ? 16 : zt >= 8 ? 8 : zt >= 4 ? 4 : zt >= 2 ? 2 : 1;
  sh.lds = config().zig_lds && sh.tiles > 1;
  return sh;
}

template <bool kFused, bool kPhilox>
static void launch_table_pass(const ZigShape &sh, const ZigArgs &a, hipStream_t stream) {
  const bool lds = sh.lds;
  switch (sh.tiles) {
    case 2:
      lds ? launch_table_pass<256, 2, true, kFused, kPhilox>(a, stream)
          : launch_table_pass<256, 2, false, kFused, kPhilox>(a, stream);
      break;
    case 4:
      lds ? launch_table_pass<256, 4, true, kFused, kPhilox>(a, stream)
          : launch_table_pass<256, 4, false, kFused, kPhilox>(a, stream);
      break;
    case 8:
      lds ? launch_table_pass<256, 8, true, kFused, kPhilox>(a, stream)
          : launch_table_pass<256, 8, false, kFused, kPhilox>(a, stream);
      break;
    case 16:
      lds ? launch_table_pass<256, 16, true, kFused, kPhilox>(a, stream)
          : launch_table_pass<256, 16, false, kFused, kPhilox>(a, stream);
      break;
    default: launch_table_pass<256, 1, false, kFused, kPhilox>(a, stream); break;
  }
}

static uint32_t zig_slot_entries(const ZigShape &sh) { return zig_slot_entries(kBlock, sh.tiles); }

// Validates and runs one f64 normal fill; the caller has set the source fields of `a`.
// Element indices within one call are 32-bit (the miss queues hold them).
template <bool kPhilox>
static tk_status normal_f64_fill(ZigArgs a, uint64_t start_draw, uint64_t n, uint64_t max_draw, double *out,
                                 hipStream_t stream) {
  if (n == 0) return TK_OK;
  if (!out || ((uintptr_t)out & 7u)) return TK_EINVAL;
  if (start_draw > max_draw || n - 1 > max_draw - start_draw) return TK_ERANGE;
  if (n > 0xFFFFFFFFull) return TK_EINVAL;
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;

  a.r = TK_ZIG_R;
  bool fused = config().zig_fused;
  bool counted = false;  // per-group miss counts kept for tk_debug_last_miss_count
  {
    std::lock_guard<std::mutex> lock(g_cap_mutex);
    if (g_debug_mode) {
      fused = g_debug_mode == 2;
      counted = true;
    }
  }
  // The two-kernel path shares the per-device lists and counters between fills (its
  // per-group counts are always kept), and a counted fused fill the count array: such
  // fills are ordered by the device's event.  The default fused fill reads only the
  // constant layer tables, so it shares nothing mutable and enqueues its kernel alone (an
  // event record per fill left ~6 us idle after each 2^28-element fill on MI355X).
  if (!fused) counted = true;
  const bool shared = counted;
  const ZigShape sh = zig_shape();
  const uint64_t per_group = (uint64_t)sh.block * sh.tiles;  // 16-byte vectors per group
  uint64_t groups = 0;
  auto geometry = [&](double *o, uint64_t s, uint64_t m) {
    a.out = o;
    a.start = s;
    a.n = m;
    a.head = ((uintptr_t)o & 15u) ? 1 : 0;
    if (a.head > m) a.head = m;
    a.nvec = (m - a.head) / 2;
    a.tail = (uint32_t)(m - a.head - 2 * a.nvec);
    groups = (a.nvec + per_group - 1) / per_group;
    if (groups == 0) groups = 1;
    a.ngroups = (uint32_t)groups;
  };
  // An output that does not start on a 4 KiB boundary would leave every work-group's
  // span across two of them, which stores slower (the streaming fills measured up to
  // 40 % slower).  The default fill then runs as two launches, the elements before the
  // first boundary and the rest (a fill cut at any element equals the whole fill).
  const uint64_t mis = (uint64_t)((uintptr_t)out & 4095u);
  const uint64_t split = (!shared && mis) ? (4096 - mis) / sizeof(double) : 0;
  geometry(out, start_draw, split && split < n ? split : n);
  a.slot_size = zig_slot_entries(sh);
  uint64_t ovf_cap = kOvfDefault;
  {
    std::lock_guard<std::mutex> lock(g_cap_mutex);
    a.slot_cap = g_debug_slot_cap ? g_debug_slot_cap : a.slot_size;
    if (g_debug_ovf_cap) ovf_cap = g_debug_ovf_cap;
  }
  a.ovf_cap = (uint32_t)ovf_cap;

  ZigDevice &d = g_zig[dev];
  std::lock_guard<std::mutex> lock(d.m);
  if ((st = zig_init(d)) != TK_OK) return st;
  if (shared) {
    if ((st = zig_reserve(d, groups, fused ? 0 : groups * a.slot_size, fused ? 0 : ovf_cap)) != TK_OK) return st;
    if (d.recorded && (st = hip_status(hipStreamWaitEvent(stream, d.last, 0))) != TK_OK) return st;
  }
  a.xx = d.xx;
  a.f = d.f;
  a.counts = shared ? d.counts : nullptr;
  a.slots = d.slots;
  a.ovf = d.ovf;
  a.ctr = d.ctr;

  if (fused) {
    launch_table_pass<true, kPhilox>(sh, a, stream);
    if ((st = launch_status()) != TK_OK) return st;
    if (split && split < n) {
      geometry(out + split, start_draw + split, n - split);
      launch_table_pass<true, kPhilox>(sh, a, stream);
      if ((st = launch_status()) != TK_OK) return st;
    }
  } else {
    hipLaunchKernelGGL(k_zig_reset, dim3(1), dim3(64), 0, stream, d.ctr);
    if ((st = launch_status()) != TK_OK) return st;
    launch_table_pass<false, kPhilox>(sh, a, stream);
    if ((st = launch_status()) != TK_OK) return st;
    // table-pass groups per continuation block: about 256 tiles of 256 lanes' worth
    uint32_t gpb = (uint32_t)(kBlock * kBlock / (sh.block * sh.tiles));
    if (gpb == 0) gpb = 1;
    const uint64_t cgrid = (groups + gpb - 1) / gpb;
    hipLaunchKernelGGL(k_zig_continue<kPhilox>, dim3((uint32_t)cgrid), dim3(kBlock), 0, stream, a, gpb);
    if ((st = launch_status()) != TK_OK) return st;
  }
  d.last_counted = counted;
  if (!shared) return TK_OK;
  if ((st = hip_status(hipEventRecord(d.last, stream))) != TK_OK) return st;
  d.recorded = true;
  d.last_groups = groups;
  d.last_fused = fused;
  return TK_OK;
}

// ---------------------------------------------------------------------------------------
// The f64 normal fill without allocation: the two-kernel path with its layer tables
// compiled into device memory and its miss lists in one static device array
// ---------------------------------------------------------------------------------------
// Largest n per call, and the shape the scratch array is sized for: 256-lane table-pass
// groups of 4 tiles (2048 elements each), whatever the launch tunables say.
constexpr uint64_t kNoAllocMaxN = 1ull << 24;
constexpr int kNoAllocTiles = 4;
constexpr uint64_t kNoAllocGroups = (kNoAllocMaxN / 2 + kBlock * kNoAllocTiles - 1) / (kBlock * kNoAllocTiles);
constexpr uint64_t kNoAllocSlot = zig_slot_entries(kBlock, kNoAllocTiles);  // entries per group
constexpr uint64_t kNoAllocOvf = 65536;                                     // overflow entries
// Layout in 32-bit words: the overflow counter (alone in the first 256 bytes), the per-group
// miss counts, the per-group slots, the overflow list: 598080 words, 2.28 MiB per device.
constexpr uint64_t kNoAllocCountsAt = 64;
constexpr uint64_t kNoAllocSlotsAt = kNoAllocCountsAt + kNoAllocGroups;
constexpr uint64_t kNoAllocOvfAt = kNoAllocSlotsAt + kNoAllocGroups * kNoAllocSlot;
constexpr uint64_t kNoAllocWords = kNoAllocOvfAt + kNoAllocOvf;
static_assert(kNoAllocCountsAt * 4 % 256 == 0 && kNoAllocSlotsAt % 64 == 0 && kNoAllocOvfAt % 64 == 0,
              "each list starts on a 256-byte boundary");

// Per-device copies (the code object is loaded on every device the library runs on, and
// each holds its own arrays until the process ends).  Host code never uses these names as
// addresses: it asks the runtime for each device's address once (hipGetSymbolAddress).
static __device__ __align__(256) uint32_t scratch[kNoAllocWords];
struct alignas(16) ZigPairRow {
  double x, y;
};
static __device__ __align__(256) ZigPairRow zig_pairs_static[TK_ZIG_LAYERS] = {TK_ZIG_PAIR_ROWS};
static __device__ __align__(256) double zig_f_static[TK_ZIG_LAYERS + 1] = {TK_ZIG_F_ROWS};

struct NoAllocDevice {
  std::mutex m;
  bool ready = false;
  uint32_t *scratch = nullptr;  // this device's `scratch`
  const double2 *xx = nullptr;  // this device's `zig_pairs_static`
  const double *f = nullptr;    // this device's `zig_f_static`
};
static NoAllocDevice g_no_alloc[kMaxDevices];

// The device addresses of the static arrays on the current device, looked up on the
// device's first call (with the device current) and kept.
static tk_status no_alloc_init(NoAllocDevice &d) {
  if (d.ready) return TK_OK;
  void *p = nullptr, *px = nullptr, *pf = nullptr;
  tk_status st;
  if ((st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))) != TK_OK) return st;
  if ((st = hip_status(hipGetSymbolAddress(&px, HIP_SYMBOL(zig_pairs_static)))) != TK_OK) return st;
  if ((st = hip_status(hipGetSymbolAddress(&pf, HIP_SYMBOL(zig_f_static)))) != TK_OK) return st;
  if (!p || !px || !pf) return TK_EHIP;
  d.scratch = (uint32_t *)p;
  d.xx = (const double2 *)px;
  d.f = (const double *)pf;
  d.ready = true;
  return TK_OK;
}

static tk_status normal_f64_no_alloc(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  if (n == 0) return TK_OK;
  if (!out || ((uintptr_t)out & 7u)) return TK_EINVAL;
  if (n > kNoAllocMaxN) return TK_EINVAL;
  if (start_draw > 0x7FFFFFFFull || n - 1 > 0x7FFFFFFFull - start_draw) return TK_ERANGE;
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;
  NoAllocDevice &d = g_no_alloc[dev];
  {
    std::lock_guard<std::mutex> lock(d.m);
    if ((st = no_alloc_init(d)) != TK_OK) return st;
  }
  ZigArgs a{};
  a.hk = host_lowbias32(key);
  a.hkp = host_substream_key(key, kPurposeNormal64);
  a.r = TK_ZIG_R;
  a.out = out;
  a.start = start_draw;
  a.n = n;
  a.head = ((uintptr_t)out & 15u) ? 1 : 0;
  a.nvec = (n - a.head) / 2;
  a.tail = (uint32_t)(n - a.head - 2 * a.nvec);
  uint64_t groups = (a.nvec + kBlock * kNoAllocTiles - 1) / (kBlock * kNoAllocTiles);
  if (groups == 0) groups = 1;
  if (groups > kNoAllocGroups) return TK_EINVAL;  // not reached for n <= kNoAllocMaxN
  a.ngroups = (uint32_t)groups;
  a.slot_size = (uint32_t)kNoAllocSlot;
  a.slot_cap = (uint32_t)kNoAllocSlot;
  a.ovf_cap = (uint32_t)kNoAllocOvf;
  a.xx = d.xx;
  a.f = d.f;
  a.ctr = d.scratch;
  a.counts = d.scratch + kNoAllocCountsAt;
  a.slots = d.scratch + kNoAllocSlotsAt;
  a.ovf = d.scratch + kNoAllocOvfAt;
  // the overflow count must start at zero (a kernel, not a memset: graph capture records
  // no memset node); the per-group counts and slots are written by every table-pass group
  hipLaunchKernelGGL(k_zig_reset, dim3(1), dim3(64), 0, stream, a.ctr);
  if ((st = launch_status()) != TK_OK) return st;
  launch_table_pass<kBlock, kNoAllocTiles, true, false, false>(a, stream);
  if ((st = launch_status()) != TK_OK) return st;
  const uint32_t gpb = (uint32_t)(kBlock * kBlock / (kBlock * kNoAllocTiles));
  const uint64_t cgrid = (groups + gpb - 1) / gpb;
  hipLaunchKernelGGL(k_zig_continue<false>, dim3((uint32_t)cgrid), dim3(kBlock), 0, stream, a, gpb);
  return launch_status();
}

}  // namespace tk

using namespace tk;

extern "C" {

tk_status tk_fill_normal_f64_no_alloc(uint32_t key, uint64_t start_draw, uint64_t n, double *out,
                                      hipStream_t stream) {
  return normal_f64_no_alloc(key, start_draw, n, out, stream);
}

tk_status tk_fill_normal_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  ZigArgs a{};
  a.hk = host_lowbias32(key);
  a.hkp = host_substream_key(key, kPurposeNormal64);
  return normal_f64_fill<false>(a, start_draw, n, 0x7FFFFFFFull, out, stream);
}

tk_status tk_philox_fill_normal_f64(uint64_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  ZigArgs a{};
  a.k0 = (uint32_t)key;
  a.k1 = (uint32_t)(key >> 32);
  return normal_f64_fill<true>(a, start_draw, n, 0x7FFFFFFFFFFFFFFFull, out, stream);
}

tk_status tk_ziggurat_table(double *x, double *f) {
  if (!x || !f) return TK_EINVAL;
  for (int i = 0; i <= TK_ZIG_LAYERS; ++i) {
    x[i] = tk_zig_x[i];
    f[i] = tk_zig_f[i];
  }
  return TK_OK;
}

tk_status tk_debug_set_miss_capacity(uint32_t per_group, uint64_t overflow) {
  if (per_group > kSlotPerTile || overflow > 0xFFFFFFFFull) return TK_EINVAL;
  std::lock_guard<std::mutex> lock(g_cap_mutex);
  g_debug_slot_cap = per_group;
  g_debug_ovf_cap = overflow;
  return TK_OK;
}

tk_status tk_debug_set_normal_f64_mode(uint32_t mode) {
  if (mode > 2) return TK_EINVAL;
  std::lock_guard<std::mutex> lock(g_cap_mutex);
  g_debug_mode = (int)mode;
  return TK_OK;
}

tk_status tk_debug_last_miss_count(uint64_t *count) {
  if (!count) return TK_EINVAL;
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;
  ZigDevice &d = g_zig[dev];
  std::lock_guard<std::mutex> lock(d.m);
  if (!d.ready) {  // no fill on this device yet
    *count = 0;
    return TK_OK;
  }
  if (!d.last_counted || !d.recorded) return TK_EINVAL;  // the last fill kept no counts
  if ((st = hip_status(hipEventSynchronize(d.last))) != TK_OK) return st;
  // every miss sits in a group's count or, in the two-kernel mode, in the overflow count
  std::vector<uint32_t> v(d.last_groups);
  if ((st = hip_status(hipMemcpy(v.data(), d.counts, v.size() * sizeof(uint32_t), hipMemcpyDeviceToHost))) != TK_OK)
    return st;
  uint32_t ovf = 0;
  if (!d.last_fused &&
      (st = hip_status(hipMemcpy(&ovf, d.ctr, sizeof(uint32_t), hipMemcpyDeviceToHost))) != TK_OK)
    return st;
  uint64_t total = ovf;
  for (uint32_t x : v) total += x;
  *count = total;
  return TK_OK;
}

}  // extern "C"
