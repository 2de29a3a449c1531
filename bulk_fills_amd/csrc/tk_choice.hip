// tk_choice.hip -- weighted choice through an alias table.
//
// tandem-sycl, "Design", §Fills: the choice fill maps each 64-bit draw through an alias
// table.  The table is built once on the host (Vose's method in integers, so it is exact
// and reproducible) and uploaded as n pairs {q, alias}.  The fill keeps the table in LDS
// (one copy per work-group of a few 4 KiB tiles) and maps draw d to column
// c = (hi32(d) n) >> 32, coin lo32(d): out = coin < q[c] ? c : alias[c].  Four indices
// leave as one 16-byte store.
#include <math.h>

#include <deque>
#include <memory>
#include <new>
#include <vector>

#include "tk_device.h"
#include "tk_internal.h"

struct tk_alias {
  int device;
  uint32_t n;
  uint2 *table;  // device: {q, alias} per column
  std::vector<uint32_t> q, alias;
};

namespace tk {

constexpr uint32_t kChoiceLdsMax = 8192;  // columns kept in LDS (64 KiB); larger tables are read from L2

// Vose's alias construction over integer masses.  Index j owns
// m_j = floor(w_j / S * n 2^32) of the n 2^32 total; the rounding remainder goes to the
// largest weight (first on ties).  Columns are filled from two FIFO lists in index order:
// an under-full index takes the front over-full one as its alias, which gives up the
// difference and rejoins the under-full list once below 2^32.
static bool build_alias(const double *w, uint32_t n, std::vector<uint32_t> &q, std::vector<uint32_t> &alias) {
  double total_w = 0.0;
  for (uint32_t j = 0; j < n; ++j) {
    if (!(w[j] >= 0.0) || !std::isfinite(w[j])) return false;
    total_w += w[j];
  }
  if (!(total_w > 0.0) || !std::isfinite(total_w)) return false;
  const uint64_t full = 1ull << 32;
  const uint64_t total = (uint64_t)n << 32;
  std::vector<uint64_t> mass(n);
  uint64_t assigned = 0;
  uint32_t biggest = 0;
  for (uint32_t j = 0; j < n; ++j) {
    mass[j] = (uint64_t)std::floor(w[j] / total_w * (double)total);
    assigned += mass[j];
    if (w[j] > w[biggest]) biggest = j;
  }
  mass[biggest] = (uint64_t)((int64_t)mass[biggest] + ((int64_t)total - (int64_t)assigned));
  q.assign(n, 0);
  alias.resize(n);
  std::deque<uint32_t> under, over;
  for (uint32_t j = 0; j < n; ++j) (mass[j] < full ? under : over).push_back(j);
  while (!under.empty() && !over.empty()) {
    const uint32_t s = under.front();
    under.pop_front();
    const uint32_t l = over.front();
    q[s] = (uint32_t)mass[s];
    alias[s] = l;
    mass[l] -= full - mass[s];
    if (mass[l] < full) {
      over.pop_front();
      under.push_back(l);
    }
  }
  for (uint32_t j : over) { q[j] = 0; alias[j] = j; }   // exactly full columns
  for (uint32_t j : under) { q[j] = 0; alias[j] = j; }  // unreachable with exact masses
  return true;
}

struct ChoiceArgs {
  uint32_t *out;
  uint64_t start, head, nvec;
  uint32_t tail;
  uint32_t hk;      // lowbias32 source: hash of the key
  uint32_t k0, k1;  // Philox source: the key
  uint32_t n;
  const uint2 *table;
};

template <bool kLds>
__device__ __forceinline__ uint32_t choose(const ChoiceArgs &a, const uint2 *tab, uint32_t lo, uint32_t hi) {
  const uint32_t col = __umulhi(hi, a.n);
  const uint2 e = kLds ? tab[col] : a.table[col];
  return lo < e.x ? col : e.y;
}

template <bool kLds, bool kPhilox>
__device__ __forceinline__ uint32_t choice_elem(const ChoiceArgs &a, const uint2 *tab, uint64_t k) {
  if (kPhilox) {
    const uint64_t w = 2 * (a.start + k);
    return choose<kLds>(a, tab, philox_word(w, a.k0, a.k1), philox_word(w + 1, a.k0, a.k1));
  }
  const uint32_t c = 2u * (uint32_t)(a.start + k);
  return choose<kLds>(a, tab, word(a.hk, c), word(a.hk, c + 1));
}

// The eight Philox words w0 .. w0+7 of a lane whose neighbour starts at w0 + 8 (word
// offset w0 & 3 is 0 or 2, the same for every lane).  At offset 2 the last two words are
// the first two of the next lane's block, handed over by from_next_lane (a DPP shift);
// lane 63 computes them.  Every lane of the wave must call this.
__device__ __forceinline__ void philox_words8(uint64_t w0, uint32_t k0, uint32_t k1, uint32_t w[8]) {
  const uint64_t b = w0 >> 2;
  const U32x4 B0 = philox4x32_10(b, k0, k1), B1 = philox4x32_10(b + 1, k0, k1);
  if ((w0 & 3u) == 0) {
    w[0] = B0.a; w[1] = B0.b; w[2] = B0.c; w[3] = B0.d;
    w[4] = B1.a; w[5] = B1.b; w[6] = B1.c; w[7] = B1.d;
    return;
  }
  uint32_t n0 = from_next_lane(B0.a), n1 = from_next_lane(B0.b);
  if (lane_id() == 63) {
    const U32x4 B2 = philox4x32_10(b + 2, k0, k1);
    n0 = B2.a; n1 = B2.b;
  }
  w[0] = B0.c; w[1] = B0.d; w[2] = B1.a; w[3] = B1.b;
  w[4] = B1.c; w[5] = B1.d; w[6] = n0; w[7] = n1;
}

// Vector v: four indices from the eight words c0 .. c0+7, c0 = 2 (start + head + 4v).  When
// start + head is a multiple of 4, c0 is a multiple of 8 and (c0 + j) ^ hk = c0 ^ (hk ^ j).
// Philox: the same four draws from Philox words 2 (start + head + 4v) ...; the whole wave
// computes its words before the range check, since the hand-over needs every lane.
template <bool kLds, bool kAligned8, bool kCheck, bool kNT, bool kPhilox>
__device__ __forceinline__ void choice_vec(const ChoiceArgs &a, const uint2 *tab, uint64_t v) {
  uint32_t r[4];
  if (kPhilox) {
    uint32_t w[8];
    philox_words8(2 * (a.start + a.head + 4 * v), a.k0, a.k1, w);
    if (kCheck && v >= a.nvec) return;
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) r[j] = choose<kLds>(a, tab, w[2 * j], w[2 * j + 1]);
  } else {
    if (kCheck && v >= a.nvec) return;
    const uint32_t c0 = 2u * (uint32_t)(a.start + a.head + 4 * v);
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
      const uint32_t lo = kAligned8 ? lowbias32(c0 ^ (a.hk ^ (2 * j))) : word(a.hk, c0 + 2 * j);
      const uint32_t hi = kAligned8 ? lowbias32(c0 ^ (a.hk ^ (2 * j + 1))) : word(a.hk, c0 + 2 * j + 1);
      r[j] = choose<kLds>(a, tab, lo, hi);
    }
  }
  store16<kNT>(a.out + a.head + 4 * v, make_uint4(r[0], r[1], r[2], r[3]));
}

template <int T, bool kLds, bool kAligned8, bool kNT, bool kPhilox>
__device__ __forceinline__ void choice_tiles(const ChoiceArgs &a, const uint2 *tab) {
  const uint64_t v0 = (uint64_t)blockIdx.x * T * kBlock + threadIdx.x;
  if ((uint64_t)(blockIdx.x + 1) * T * kBlock <= a.nvec) {
    for (int t = 0; t < T; ++t) choice_vec<kLds, kAligned8, false, kNT, kPhilox>(a, tab, v0 + (uint64_t)t * kBlock);
  } else {
    for (int t = 0; t < T; ++t) choice_vec<kLds, kAligned8, true, kNT, kPhilox>(a, tab, v0 + (uint64_t)t * kBlock);
  }
}

// T consecutive 4 KiB tiles per work-group over a one-shot grid; with kLds the table is
// copied to LDS once per group.  Two tiles by default: with the direct-to-LDS copy they
// measured ~167 us at 2^28 elements on MI355X, against ~178 us for four tiles (and ~172 us
// for four tiles with the copy through registers).
template <int T, bool kLds, bool kNT, bool kPhilox>
__global__ __launch_bounds__(kBlock) void k_choice(ChoiceArgs a) {
  extern __shared__ uint2 tab[];
  if (kLds) {
    // direct-to-LDS loads (global_load_lds_dwordx4), two columns per lane: a wave's 64
    // 16-byte loads land at consecutive LDS addresses without passing through VGPRs.  The
    // device table is padded to an even number of columns, so the last load stays inside
    // it; lanes past the end are masked off.
    const uint32_t chunks = (a.n + 1) >> 1;
    const uint32_t wave_base = threadIdx.x & ~63u;
    for (uint32_t c0 = 0; c0 < chunks; c0 += kBlock) {
      if (c0 + threadIdx.x < chunks)
        __builtin_amdgcn_global_load_lds((const void *)((const uint4 *)a.table + c0 + threadIdx.x),
                                         (void *)((uint4 *)tab + c0 + wave_base), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's copies are in LDS
    __syncthreads();                          // and every other wave's
  }
  if (((a.start + a.head) & 3u) == 0) choice_tiles<T, kLds, true, kNT, kPhilox>(a, tab);
  else choice_tiles<T, kLds, false, kNT, kPhilox>(a, tab);
  if (blockIdx.x == 0) {  // the elements before the first vector (under 1024) and after the last
    for (uint64_t k = threadIdx.x; k < a.head; k += kBlock) a.out[k] = choice_elem<kLds, kPhilox>(a, tab, k);
    if (threadIdx.x < a.tail) {
      const uint64_t k = a.head + 4 * a.nvec + threadIdx.x;
      a.out[k] = choice_elem<kLds, kPhilox>(a, tab, k);
    }
  }
}

template <int T, bool kLds, bool kPhilox>
static void launch_choice_t(const ChoiceArgs &a, uint32_t grid, hipStream_t stream) {
  const int pad = config().lds_pad;  // tunable: extra dynamic LDS, which caps the groups per CU
  const size_t lds = (kLds ? (size_t)((a.n + 1) & ~1u) * sizeof(uint2) : 0) + (pad > 0 ? (size_t)pad : 0);
  if (config().nt_stores)
    hipLaunchKernelGGL((k_choice<T, kLds, true, kPhilox>), dim3(grid), dim3(kBlock), lds, stream, a);
  else
    hipLaunchKernelGGL((k_choice<T, kLds, false, kPhilox>), dim3(grid), dim3(kBlock), lds, stream, a);
}

template <bool kLds, bool kPhilox>
static void launch_choice(const ChoiceArgs &a, int tiles, hipStream_t stream) {
  const uint64_t per_group = (uint64_t)kBlock * tiles;
  uint64_t groups = (a.nvec + per_group - 1) / per_group;
  if (groups == 0) groups = 1;
  switch (tiles) {
    case 1: launch_choice_t<1, kLds, kPhilox>(a, (uint32_t)groups, stream); break;
    case 2: launch_choice_t<2, kLds, kPhilox>(a, (uint32_t)groups, stream); break;
    case 8: launch_choice_t<8, kLds, kPhilox>(a, (uint32_t)groups, stream); break;
    default: launch_choice_t<4, kLds, kPhilox>(a, (uint32_t)groups, stream); break;
  }
}

// Validates and launches a choice fill; the caller has set the source fields of `a`.
template <bool kPhilox>
static tk_status choice_fill(ChoiceArgs a, uint64_t start_draw, uint64_t n, uint64_t max_draw, const tk_alias *table,
                             uint32_t *out, hipStream_t stream) {
  if (!table) return TK_EINVAL;
  if (n == 0) return TK_OK;
  if (!out || ((uintptr_t)out & 3u)) return TK_EINVAL;
  if (start_draw > max_draw || n - 1 > max_draw - start_draw) return TK_ERANGE;
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;
  if (dev != table->device) return TK_EINVAL;
  a.out = out;
  a.start = start_draw;
  // vectors from the output's first 4 KiB boundary, as in the streaming fills: a tile that
  // spans two 4 KiB blocks stores slower; the elements before it are written singly
  const uint64_t mis = (uintptr_t)out & 4095u;
  a.head = mis ? (4096 - mis) / 4 : 0;
  if (a.head > n) a.head = n;
  a.nvec = (n - a.head) / 4;
  a.tail = (uint32_t)(n - a.head - 4 * a.nvec);
  a.n = table->n;
  a.table = table->table;
  const int zt = config().choice_tiles;
  const int tiles = zt >= 8 ? 8 : zt >= 4 ? 4 : zt >= 2 ? 2 : 1;
  if (a.n <= kChoiceLdsMax) launch_choice<true, kPhilox>(a, tiles, stream);
  else launch_choice<false, kPhilox>(a, tiles, stream);
  return launch_status();
}

// The body of tk_alias_create.  Every host allocation happens before the device one, so
// an exception from them leaves nothing behind (the handle is owned until returned).
static tk_status alias_create(const double *weights, uint32_t n, tk_alias **table) {
  std::unique_ptr<tk_alias> t(new tk_alias());
  t->n = n;
  t->table = nullptr;
  if (!build_alias(weights, n, t->q, t->alias)) return TK_EINVAL;  // weights are checked before any HIP call
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;
  t->device = dev;
  // padded to an even number of columns: the fill copies the table 16 bytes at a time
  const uint32_t padded = (n + 1) & ~1u;
  std::vector<uint2> packed(padded, make_uint2(0u, 0u));
  for (uint32_t j = 0; j < n; ++j) packed[j] = make_uint2(t->q[j], t->alias[j]);
  if (device_alloc((void **)&t->table, padded * sizeof(uint2)) != hipSuccess) return TK_ENOMEM;
  if ((st = hip_status(hipMemcpy(t->table, packed.data(), padded * sizeof(uint2), hipMemcpyHostToDevice))) != TK_OK) {
    (void)device_free(t->table, padded * sizeof(uint2));
    return st;
  }
  *table = t.release();
  return TK_OK;
}

static tk_status alias_build_host(const double *weights, uint32_t n, uint32_t *q, uint32_t *alias) {
  std::vector<uint32_t> vq, va;
  if (!build_alias(weights, n, vq, va)) return TK_EINVAL;
  for (uint32_t j = 0; j < n; ++j) {
    q[j] = vq[j];
    alias[j] = va[j];
  }
  return TK_OK;
}

}  // namespace tk

using namespace tk;

extern "C" {

tk_status tk_alias_create(const double *weights, uint32_t n, tk_alias **table) {
  if (!weights || !table || n == 0 || n > (1u << 24)) return TK_EINVAL;
  *table = nullptr;
  // the host-side construction allocates (up to a few hundred MB for 2^24 columns); a
  // failed host allocation returns TK_ENOMEM instead of leaving the C ABI as an exception
  try {
    return alias_create(weights, n, table);
  } catch (const std::bad_alloc &) {
    return TK_ENOMEM;
  }
}

tk_status tk_alias_destroy(tk_alias *t) {
  if (!t) return TK_EINVAL;
  tk_status st = TK_OK;
  if (t->table) st = hip_status(device_free(t->table, ((t->n + 1) & ~1u) * sizeof(uint2)));
  delete t;
  return st;
}

uint32_t tk_alias_size(const tk_alias *t) { return t ? t->n : 0; }

tk_status tk_alias_build_host(const double *weights, uint32_t n, uint32_t *q, uint32_t *alias) {
  if (!weights || !q || !alias || n == 0 || n > (1u << 24)) return TK_EINVAL;
  try {
    return alias_build_host(weights, n, q, alias);
  } catch (const std::bad_alloc &) {
    return TK_ENOMEM;
  }
}

tk_status tk_alias_export(const tk_alias *t, uint32_t *q, uint32_t *alias) {
  if (!t || !q || !alias) return TK_EINVAL;
  for (uint32_t j = 0; j < t->n; ++j) {
    q[j] = t->q[j];
    alias[j] = t->alias[j];
  }
  return TK_OK;
}

tk_status tk_fill_choice_u32(uint32_t key, uint64_t start_draw, uint64_t n, const tk_alias *table, uint32_t *out,
                             hipStream_t stream) {
  ChoiceArgs a{};
  a.hk = host_lowbias32(key);
  return choice_fill<false>(a, start_draw, n, 0x7FFFFFFFull, table, out, stream);
}

tk_status tk_philox_fill_choice_u32(uint64_t key, uint64_t start_draw, uint64_t n, const tk_alias *table,
                                    uint32_t *out, hipStream_t stream) {
  ChoiceArgs a{};
  a.k0 = (uint32_t)key;
  a.k1 = (uint32_t)(key >> 32);
  return choice_fill<true>(a, start_draw, n, 0x7FFFFFFFFFFFFFFFull, table, out, stream);
}

}  // extern "C"
