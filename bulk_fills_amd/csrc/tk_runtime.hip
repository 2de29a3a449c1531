// tk_runtime.hip -- status strings, per-thread error state, tunables, device queries.
#include <stdlib.h>
#include <string.h>

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

const Config &config() {
  static const Config cfg = [] {
    Config c;
    const char *st = getenv("TK_STORE");
    c.nt_stores = st && strcmp(st, "nt") == 0;
    c.max_blocks = env_u64("TK_MAX_BLOCKS", 0x7FFFFFFFull);
    c.unroll = (int)env_u64("TK_UNROLL", 1);
    c.choice_tiles = (int)env_u64("TK_CHOICE_TILES", 4);
    c.exp_tiles = (int)env_u64("TK_EXP_TILES", 2);
    c.zig_tiles = (int)env_u64("TK_ZIG_TILES", 4);
    const char *zt = getenv("TK_ZIG_TABLE");
    c.zig_lds = !(zt && strcmp(zt, "global") == 0);
    const char *zm = getenv("TK_ZIG_MODE");
    c.zig_fused = !(zm && strcmp(zm, "split") == 0);
    return c;
  }();
  return cfg;
}

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

}  // extern "C"
