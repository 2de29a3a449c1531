// tk_ziggurat.hip -- f64 normal fill: the 1024-layer ziggurat as two kernels.
//
// tandem-sycl, "Design", §Normals: element i takes 64-bit draw i; about 0.43 % of draws
// miss the fast path and continue on the per-index substream split(i) of
// sub(key, PURPOSE_NORMAL64).  Fills of any length run two kernels:
//   * the table pass writes every fast-path value with 16-byte stores (two elements per
//     lane) and collects its work-group's misses through wave ballots into an LDS queue;
//     the queue is written to the work-group's own slot of the device miss list (at most
//     kSlot entries plus a count), so no atomic is needed.  A work-group with more misses
//     than its slot holds (probability ~1e-10 per group) appends the rest to an
//     overflow list with one atomic each;
//   * the continuation pass takes the listed misses (one slot per lane) and finishes
//     each on its substream: the wedge test against exp(-x^2/2), or the tail beyond r.
//     If the overflow list itself overflowed it walks the whole fill instead, so the
//     result never depends on the list sizes.
// The fast path makes no calls, so its register footprint stays that of a streaming fill.
// The 16 KiB layer table (pairs {X[L], X[L+1]}) lives in device memory and is read
// through the vector caches: divergent layer reads would serialize in scalar/constant
// memory (the page measured a drop to 27 GiB/s that way).  The table, the lists and the
// counters are per-device state shared by all streams; fills wait on the previous
// fill's event before touching them.
//
// The pages' design appends each group's misses with one atomic add; with the one-shot
// grid that streams fastest on MI355X (one 4 KiB tile per group, about half a million
// groups at 2^28 elements) that would put half a million atomics on one address, so each
// group owns a slot instead.
#include <math.h>

#include <mutex>

#include "tk_device.h"
#include "tk_internal.h"
#include "zig1024.inc"

namespace tk {

constexpr uint32_t kSlot = 16;  // misses a work-group keeps in its own slot

struct ZigArgs {
  double *out;
  uint64_t start;  // draw of element 0
  uint64_t n;
  uint64_t head;   // 0 or 1 element before the first 16-byte boundary
  uint64_t nvec;   // whole 16-byte vectors (two elements each)
  uint32_t tail;   // 0 or 1 element after them
  uint32_t hk;     // lowbias32(key)
  uint32_t hkp;    // lowbias32(sub(key, NORM))
  const double2 *xx;  // {X[L], X[L+1]}, L < 1024
  const double *f;    // F[0 .. 1024]
  double r;
  uint32_t ngroups;    // table-pass work-groups = slots
  uint32_t slot_cap;   // entries used per slot (<= kSlot)
  uint32_t *counts;    // [ngroups] misses kept in each slot
  uint32_t *slots;     // [ngroups * kSlot]
  uint32_t *ovf;       // overflow list
  uint32_t ovf_cap;
  uint32_t *ctr;  // [0] overflow entries, [1] finished continuation blocks, [2] last miss total, [3] running total
};

// Fast path of one draw: returns true and the value when u X[L] < X[L+1].
__device__ __forceinline__ bool zig_fast(const ZigArgs &a, uint32_t lo, uint32_t hi, double *val) {
  const uint32_t L = lo & 1023u;
  const double u = unit53_topbits(lo, hi);
  const double2 e = a.xx[L];
  const double x = u * e.x;
  *val = (lo & 1024u) ? -x : x;
  return x < e.y;
}

// Appends element k to the work-group's queue for every lane with `pred`.  Called by all
// lanes of the wave.
__device__ __forceinline__ void enqueue(bool pred, uint32_t k, uint32_t *q, uint32_t *qn, const ZigArgs &a) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(qn, (uint32_t)__popcll(m));
  base = (uint32_t)__shfl((int)base, leader);
  if (pred) {
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint32_t slot = base + rank;
    if (slot < a.slot_cap) {
      q[slot] = k;
    } else {  // the group's slot is full: overflow list
      const uint32_t g = atomicAdd(&a.ctr[0], 1u);
      if (g < a.ovf_cap) a.ovf[g] = k;
    }
  }
}

template <int U, bool kNT>
__global__ __launch_bounds__(kBlock) void k_zig_table_pass(ZigArgs a) {
  __shared__ uint32_t q[kSlot];
  __shared__ uint32_t qn;
  if (threadIdx.x == 0) qn = 0;
  __syncthreads();
  const uint64_t v0 = (uint64_t)blockIdx.x * (kBlock * U) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t v = v0 + (uint64_t)u * kBlock;
    const bool in = v < a.nvec;
    const uint32_t c = 2u * (uint32_t)(a.start + a.head + 2 * v);
    double y0, y1;
    const bool f0 = zig_fast(a, word(a.hk, c), word(a.hk, c + 1), &y0);
    const bool f1 = zig_fast(a, word(a.hk, c + 2), word(a.hk, c + 3), &y1);
    if (in) {
      uint4 w;
      w.x = (uint32_t)__double_as_longlong(y0);
      w.y = (uint32_t)((uint64_t)__double_as_longlong(y0) >> 32);
      w.z = (uint32_t)__double_as_longlong(y1);
      w.w = (uint32_t)((uint64_t)__double_as_longlong(y1) >> 32);
      store16<kNT>(a.out + a.head + 2 * v, w);
    }
    const uint32_t k0 = (uint32_t)(a.head + 2 * v);
    enqueue(in && !f0, k0, q, &qn, a);
    enqueue(in && !f1, k0 + 1, q, &qn, a);
  }
  if (blockIdx.x == 0) {  // the element before the first boundary and the one after the last vector
    const uint32_t t = threadIdx.x;
    bool edge = false;
    uint64_t k = 0;
    if (t == 0 && a.head) { edge = true; k = 0; }
    if (t == 64 && a.tail) { edge = true; k = a.head + 2 * a.nvec; }
    bool fast = true;
    if (edge) {
      const uint32_t c = 2u * (uint32_t)(a.start + k);
      double y;
      fast = zig_fast(a, word(a.hk, c), word(a.hk, c + 1), &y);
      a.out[k] = y;
    }
    enqueue(edge && !fast, (uint32_t)k, q, &qn, a);
  }
  __syncthreads();
  const uint32_t nq = qn < a.slot_cap ? qn : a.slot_cap;
  if (threadIdx.x == 0) a.counts[blockIdx.x] = nq;
  if (threadIdx.x < nq) a.slots[(uint64_t)blockIdx.x * kSlot + threadIdx.x] = q[threadIdx.x];
}

// Finishes the draw of element k from its primary draw: wedge, tail and restarts all read
// the substream split(start + k) in order.
__device__ double zig_slow(const ZigArgs &a, uint64_t k) {
  const uint32_t i = (uint32_t)(a.start + k);
  uint32_t lo = word(a.hk, 2u * i), hi = word(a.hk, 2u * i + 1u);
  Substream ss(a.hkp, i);
  const uint32_t cap_words = 2u * kSubstreamCap;
  for (;;) {
    const uint32_t L = lo & 1023u;
    const bool neg = (lo & 1024u) != 0;
    const double2 e = a.xx[L];
    const double x = unit53_topbits(lo, hi) * e.x;
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

__global__ __launch_bounds__(kBlock) void k_zig_continue(ZigArgs a) {
  __shared__ uint32_t s_ovf, s_total;
  if (threadIdx.x == 0) {
    s_ovf = __hip_atomic_load(&a.ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_total = 0;
  }
  __syncthreads();
  const uint32_t ovf = s_ovf;
  const uint64_t gid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  uint32_t mine = 0;
  if (ovf <= a.ovf_cap) {
    for (uint64_t b = gid; b < a.ngroups; b += stride) {
      const uint32_t cnt = a.counts[b];
      mine += cnt;
      for (uint32_t j = 0; j < cnt; ++j) {
        const uint32_t k = a.slots[b * kSlot + j];
        a.out[k] = zig_slow(a, k);
      }
    }
    for (uint64_t j = gid; j < ovf; j += stride) {
      const uint32_t k = a.ovf[j];
      a.out[k] = zig_slow(a, k);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) mine += ovf;
  } else {  // the overflow list overflowed: find the misses by walking the whole fill
    for (uint64_t k = gid; k < a.n; k += stride) {
      const uint32_t c = 2u * (uint32_t)(a.start + k);
      double y;
      if (!zig_fast(a, word(a.hk, c), word(a.hk, c + 1), &y)) {
        a.out[k] = zig_slow(a, k);
        ++mine;
      }
    }
  }
  if (mine) atomicAdd(&s_total, mine);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_total) atomicAdd(&a.ctr[3], s_total);
    __threadfence();
    const uint32_t done = atomicAdd(&a.ctr[1], 1u);
    if (done == gridDim.x - 1) {  // every block has read the overflow count: reset for the next fill
      const uint32_t total = __hip_atomic_load(&a.ctr[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctr[2], total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctr[3], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
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
  uint64_t groups_cap = 0;  // slots allocated
  uint32_t *ovf = nullptr;
  uint64_t ovf_alloc = 0;
  hipEvent_t last = nullptr;
  bool recorded = false;
};

static ZigDevice g_zig[kMaxDevices];
static std::mutex g_cap_mutex;
static uint32_t g_debug_slot_cap = 0;
static uint64_t g_debug_ovf_cap = 0;
constexpr uint64_t kOvfDefault = 65536;

static tk_status zig_init(ZigDevice &d) {
  if (d.ready) return TK_OK;
  double2 pairs[TK_ZIG_LAYERS];
  for (int L = 0; L < TK_ZIG_LAYERS; ++L) pairs[L] = make_double2(tk_zig_x[L], tk_zig_x[L + 1]);
  if (hipMalloc(&d.xx, sizeof(pairs)) != hipSuccess) return TK_ENOMEM;
  if (hipMalloc(&d.f, sizeof(tk_zig_f)) != hipSuccess) return TK_ENOMEM;
  if (hipMalloc(&d.ctr, 4 * sizeof(uint32_t)) != hipSuccess) return TK_ENOMEM;
  tk_status st;
  if ((st = hip_status(hipMemcpy(d.xx, pairs, sizeof(pairs), hipMemcpyHostToDevice))) != TK_OK) return st;
  if ((st = hip_status(hipMemcpy(d.f, tk_zig_f, sizeof(tk_zig_f), hipMemcpyHostToDevice))) != TK_OK) return st;
  if ((st = hip_status(hipMemset(d.ctr, 0, 4 * sizeof(uint32_t)))) != TK_OK) return st;
  if ((st = hip_status(hipEventCreateWithFlags(&d.last, hipEventDisableTiming))) != TK_OK) return st;
  d.ready = true;
  return TK_OK;
}

// Grows the slot arrays and the overflow list; the previous fill may still read them, so
// it is waited for first.
static tk_status zig_reserve(ZigDevice &d, uint64_t groups, uint64_t ovf_cap) {
  if (groups <= d.groups_cap && ovf_cap <= d.ovf_alloc) return TK_OK;
  tk_status st;
  if (d.recorded && (st = hip_status(hipEventSynchronize(d.last))) != TK_OK) return st;
  if (groups > d.groups_cap) {
    if (d.counts) (void)hipFree(d.counts);
    if (d.slots) (void)hipFree(d.slots);
    d.counts = d.slots = nullptr;
    d.groups_cap = 0;
    if (hipMalloc(&d.counts, groups * sizeof(uint32_t)) != hipSuccess) return TK_ENOMEM;
    if (hipMalloc(&d.slots, groups * kSlot * sizeof(uint32_t)) != hipSuccess) return TK_ENOMEM;
    d.groups_cap = groups;
  }
  if (ovf_cap > d.ovf_alloc) {
    if (d.ovf) (void)hipFree(d.ovf);
    d.ovf = nullptr;
    d.ovf_alloc = 0;
    if (hipMalloc(&d.ovf, ovf_cap * sizeof(uint32_t)) != hipSuccess) return TK_ENOMEM;
    d.ovf_alloc = ovf_cap;
  }
  return TK_OK;
}

template <int U>
static void launch_table_pass(const ZigArgs &a, hipStream_t stream) {
  if (config().nt_stores)
    hipLaunchKernelGGL((k_zig_table_pass<U, true>), dim3(a.ngroups), dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((k_zig_table_pass<U, false>), dim3(a.ngroups), dim3(kBlock), 0, stream, a);
}

}  // namespace tk

using namespace tk;

extern "C" {

tk_status tk_fill_normal_f64(uint32_t key, uint64_t start_draw, uint64_t n, double *out, hipStream_t stream) {
  if (n == 0) return TK_OK;
  if (!out || ((uintptr_t)out & 7u)) return TK_EINVAL;
  if (start_draw > 0x7FFFFFFFull || n - 1 > 0x7FFFFFFFull - start_draw) return TK_ERANGE;
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;

  ZigArgs a{};
  a.out = out;
  a.start = start_draw;
  a.n = n;
  a.head = ((uintptr_t)out & 15u) ? 1 : 0;
  if (a.head > n) a.head = n;
  a.nvec = (n - a.head) / 2;
  a.tail = (uint32_t)(n - a.head - 2 * a.nvec);
  a.hk = host_lowbias32(key);
  a.hkp = host_substream_key(key, kPurposeNormal64);
  a.r = TK_ZIG_R;
  const int U = config().unroll == 2 ? 2 : 1;
  const uint64_t per_group = (uint64_t)kBlock * U;
  uint64_t groups = (a.nvec + per_group - 1) / per_group;
  if (groups == 0) groups = 1;
  a.ngroups = (uint32_t)groups;
  uint64_t ovf_cap = kOvfDefault;
  {
    std::lock_guard<std::mutex> lock(g_cap_mutex);
    a.slot_cap = g_debug_slot_cap ? g_debug_slot_cap : kSlot;
    if (g_debug_ovf_cap) ovf_cap = g_debug_ovf_cap;
  }
  a.ovf_cap = (uint32_t)ovf_cap;

  ZigDevice &d = g_zig[dev];
  std::lock_guard<std::mutex> lock(d.m);
  if ((st = zig_init(d)) != TK_OK) return st;
  if ((st = zig_reserve(d, groups, ovf_cap)) != TK_OK) return st;
  if (d.recorded && (st = hip_status(hipStreamWaitEvent(stream, d.last, 0))) != TK_OK) return st;
  a.xx = d.xx;
  a.f = d.f;
  a.counts = d.counts;
  a.slots = d.slots;
  a.ovf = d.ovf;
  a.ctr = d.ctr;

  if (U == 2) launch_table_pass<2>(a, stream);
  else launch_table_pass<1>(a, stream);
  if ((st = launch_status()) != TK_OK) return st;

  uint64_t cgrid = (groups + kBlock - 1) / kBlock;
  if (cgrid > 4096) cgrid = 4096;
  hipLaunchKernelGGL(k_zig_continue, dim3((uint32_t)cgrid), dim3(kBlock), 0, stream, a);
  if ((st = launch_status()) != TK_OK) return st;
  if ((st = hip_status(hipEventRecord(d.last, stream))) != TK_OK) return st;
  d.recorded = true;
  return TK_OK;
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
  if (per_group > kSlot || overflow > 0xFFFFFFFFull) return TK_EINVAL;
  std::lock_guard<std::mutex> lock(g_cap_mutex);
  g_debug_slot_cap = per_group;
  g_debug_ovf_cap = overflow;
  return TK_OK;
}

tk_status tk_debug_last_miss_count(uint64_t *count) {
  if (!count) return TK_EINVAL;
  tk_status st;
  const int dev = current_device(&st);
  if (dev < 0) return st;
  ZigDevice &d = g_zig[dev];
  std::lock_guard<std::mutex> lock(d.m);
  if (!d.ready || !d.recorded) {
    *count = 0;
    return TK_OK;
  }
  if ((st = hip_status(hipEventSynchronize(d.last))) != TK_OK) return st;
  uint32_t v = 0;
  if ((st = hip_status(hipMemcpy(&v, d.ctr + 2, sizeof(v), hipMemcpyDeviceToHost))) != TK_OK) return st;
  *count = v;
  return TK_OK;
}

}  // extern "C"
