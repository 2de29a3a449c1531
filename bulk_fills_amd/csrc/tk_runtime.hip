// tk_runtime.hip -- status strings, per-thread error state, tunables, device queries.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "tk_internal.h"

namespace tk {

static thread_local int g_last_hip_error = 0;

void set_hip_error(hipError_t e) { g_last_hip_error = (int)e; }

static uint64_t env_u64(const char *name, uint64_t dflt) {
  const char *s = getenv(name);
  if (!s || !*s) return dflt;
  char *end = nullptr;
  unsigned long long v = strtoull(s, &end, 10);
  return (end && *end == 0 && v > 0) ? (uint64_t)v : dflt;
}

// Sets one tunable from the environment (the defaults when a variable is unset).
static bool env_tunable(Config &c, const char *name) {
  if (!strcmp(name, "store_nt")) {
    const char *st = getenv("TK_STORE");
    c.nt_stores = st && strcmp(st, "nt") == 0;
  } else if (!strcmp(name, "max_blocks")) {
    c.max_blocks = env_u64("TK_MAX_BLOCKS", 0x7FFFFFFFull);
  } else if (!strcmp(name, "unroll")) {
    c.unroll = (int)env_u64("TK_UNROLL", 1);
  } else if (!strcmp(name, "choice_tiles")) {
    c.choice_tiles = (int)env_u64("TK_CHOICE_TILES", 2);
  } else if (!strcmp(name, "exp_tiles")) {
    c.exp_tiles = (int)env_u64("TK_EXP_TILES", 2);
  } else if (!strcmp(name, "zig_tiles")) {
    c.zig_tiles = (int)env_u64("TK_ZIG_TILES", 4);
  } else if (!strcmp(name, "zig_lds")) {
    const char *zt = getenv("TK_ZIG_TABLE");
    c.zig_lds = !(zt && strcmp(zt, "global") == 0);
  } else if (!strcmp(name, "zig_fused")) {
    const char *zm = getenv("TK_ZIG_MODE");
    c.zig_fused = !(zm && strcmp(zm, "split") == 0);
  } else if (!strcmp(name, "philox_lds")) {
    const char *ph = getenv("TK_PHILOX");
    c.philox_lds = !(ph && strcmp(ph, "overlap") == 0);
  } else if (!strcmp(name, "pair_lds")) {
    const char *pr = getenv("TK_PAIRS");
    c.pair_lds = !(pr && strcmp(pr, "wave") == 0);
  } else if (!strcmp(name, "lds_pad")) {
    const char *lp = getenv("TK_LDS_PAD");
    const uint64_t b = lp ? env_u64("TK_LDS_PAD", 0) : 0;
    c.lds_pad = !lp ? -1 : b > 65536 ? 65536 : (int)b;
  } else if (!strcmp(name, "zig_lds_pad")) {
    const uint64_t b = env_u64("TK_ZIG_LDS_PAD", 0);
    c.zig_lds_pad = b > 65536 ? 65536 : (int)b;
  } else if (!strcmp(name, "const_work")) {
    const uint64_t w = env_u64("TK_CONST_WORK", 0);
    c.const_work = w > 4096 ? 4096 : (int)w;
  } else {
    return false;
  }
  return true;
}

static const char *const kTunables[] = {"store_nt",  "max_blocks", "unroll",  "choice_tiles", "exp_tiles",
                                        "zig_tiles", "zig_lds",    "zig_fused", "philox_lds", "pair_lds",
                                        "lds_pad",   "zig_lds_pad", "const_work"};

static Config &mutable_config() {
  static Config cfg;
  static std::once_flag once;
  std::call_once(once, [] {
    for (const char *name : kTunables) env_tunable(cfg, name);
  });
  return cfg;
}

const Config &config() { return mutable_config(); }

int current_device(tk_status *st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e);
    return -1;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = TK_EINVAL;
    return -1;
  }
  *st = TK_OK;
  return dev;
}

static std::mutex g_alloc_mutex;
static uint32_t g_alloc_skip = 0;  // allocations still to succeed before the forced failures
static uint32_t g_alloc_fail = 0;  // forced failures still to come
static std::atomic<uint64_t> g_device_bytes{0};

// TK_DEBUG_FAIL_ALLOC=<n>: the process's first n device allocations fail.  Read once,
// before the first allocation or the first tk_debug_fail_allocations call, whichever
// comes first (a later call replaces it).
static void apply_env_failures() {
  static std::once_flag once;
  std::call_once(once, [] {
    const uint64_t n = env_u64("TK_DEBUG_FAIL_ALLOC", 0);
    std::lock_guard<std::mutex> lock(g_alloc_mutex);
    if (n) {
      g_alloc_fail = n > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)n;
      // said once, so that a forced TK_ENOMEM is never taken for a real one
      fprintf(stderr, "libtk: TK_DEBUG_FAIL_ALLOC=%llu is set: the first %u device allocations of this "
              "process fail with TK_ENOMEM (a test hook)\n", (unsigned long long)n, g_alloc_fail);
    }
  });
}

hipError_t device_alloc(void **p, size_t bytes) {
  *p = nullptr;
  apply_env_failures();
  {
    std::lock_guard<std::mutex> lock(g_alloc_mutex);
    if (g_alloc_skip > 0) {
      --g_alloc_skip;
    } else if (g_alloc_fail > 0) {
      --g_alloc_fail;
      return hipErrorOutOfMemory;
    }
  }
  const hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    // HIP keeps a failed call's error for hipGetLastError; clear it so that the next
    // launch's status check does not report this allocation as a launch failure
    (void)hipGetLastError();
    return e;
  }
  g_device_bytes += bytes;
  return hipSuccess;
}

hipError_t device_free(void *p, size_t bytes) {
  if (!p) return hipSuccess;
  g_device_bytes -= bytes;
  return hipFree(p);
}

int device_cus(int device) {
  static int cus[kMaxDevices];
  static std::mutex m;
  std::lock_guard<std::mutex> lock(m);
  if (cus[device] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || v <= 0) v = 256;
    cus[device] = v;
  }
  return cus[device];
}

}  // namespace tk

extern "C" {

const char *tk_status_string(tk_status s) {
  switch (s) {
    case TK_OK: return "TK_OK: success";
    case TK_EINVAL: return "TK_EINVAL: invalid argument";
    case TK_ERANGE: return "TK_ERANGE: draws outside the counter space or range does not fit the output type";
    case TK_ENOMEM: return "TK_ENOMEM: device allocation for library state failed";
    case TK_EHIP: return "TK_EHIP: HIP runtime error (see tk_last_hip_error)";
  }
  return "unknown tk_status";
}

int tk_last_hip_error(void) { return tk::g_last_hip_error; }

tk_status tk_debug_fail_allocations(uint32_t skip, uint32_t count) {
  tk::apply_env_failures();
  std::lock_guard<std::mutex> lock(tk::g_alloc_mutex);
  tk::g_alloc_skip = count ? skip : 0;
  tk::g_alloc_fail = count;
  return TK_OK;
}

tk_status tk_debug_device_bytes(uint64_t *bytes) {
  if (!bytes) return TK_EINVAL;
  *bytes = tk::g_device_bytes.load();
  return TK_OK;
}

tk_status tk_debug_set_tunable(const char *name, int64_t value) {
  using namespace tk;
  if (!name) return TK_EINVAL;
  Config &c = mutable_config();
  if (value < 0) return env_tunable(c, name) ? TK_OK : TK_EINVAL;  // back to the environment's value
  const auto one_of = [value](std::initializer_list<int64_t> ok) {
    for (int64_t v : ok)
      if (v == value) return true;
    return false;
  };
  if (!strcmp(name, "store_nt") && one_of({0, 1})) c.nt_stores = value == 1;
  else if (!strcmp(name, "max_blocks") && value >= 1 && value <= 0x7FFFFFFF) c.max_blocks = (uint64_t)value;
  else if (!strcmp(name, "unroll") && one_of({1, 2, 4})) c.unroll = (int)value;
  else if (!strcmp(name, "choice_tiles") && one_of({1, 2, 4, 8})) c.choice_tiles = (int)value;
  else if (!strcmp(name, "exp_tiles") && one_of({1, 2, 4})) c.exp_tiles = (int)value;
  else if (!strcmp(name, "zig_tiles") && one_of({1, 2, 4, 8, 16})) c.zig_tiles = (int)value;
  else if (!strcmp(name, "zig_lds") && one_of({0, 1})) c.zig_lds = value == 1;
  else if (!strcmp(name, "zig_fused") && one_of({0, 1})) c.zig_fused = value == 1;
  else if (!strcmp(name, "philox_lds") && one_of({0, 1})) c.philox_lds = value == 1;
  else if (!strcmp(name, "pair_lds") && one_of({0, 1})) c.pair_lds = value == 1;
  else if (!strcmp(name, "lds_pad") && value <= 65536) c.lds_pad = (int)value;
  else if (!strcmp(name, "zig_lds_pad") && value <= 65536) c.zig_lds_pad = (int)value;
  else if (!strcmp(name, "const_work") && value <= 4096) c.const_work = (int)value;
  else return TK_EINVAL;
  return TK_OK;
}

}  // extern "C"
