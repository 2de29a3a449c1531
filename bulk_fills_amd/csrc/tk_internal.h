// tk_internal.h -- host-side helpers shared by the libtk translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include <mutex>

#include "tk.h"
#include "tk_device_api.h"

namespace tk {

// Last HIP error seen by this thread (reported by tk_last_hip_error).
void set_hip_error(hipError_t e);

// Maps a HIP error to TK_EHIP (recording it) or TK_OK.
inline tk_status hip_status(hipError_t e) {
  if (e == hipSuccess) return TK_OK;
  set_hip_error(e);
  return TK_EHIP;
}

// Status of the most recent kernel launch on this thread.
inline tk_status launch_status() { return hip_status(hipGetLastError()); }

// The generator's hash on the host (the public API's tk_hash32, shared with the kernels).
inline uint32_t host_lowbias32(uint32_t x) { return tk_hash32(x); }

// Purpose tags of sub(key, P) (ASCII "NORM", "BL32", "BL64").
constexpr uint32_t kPurposeNormal64 = 0x4E4F524Du;
constexpr uint32_t kPurposeBelow32 = 0x424C3332u;
constexpr uint32_t kPurposeBelow64 = 0x424C3634u;

// lowbias32(sub(key, P)) with sub(key, P) = lowbias32(lowbias32(key) ^ P): the value the
// kernels need to open the substream of any draw for purpose P.
inline uint32_t host_substream_key(uint32_t key, uint32_t purpose) {
  return host_lowbias32(host_lowbias32(host_lowbias32(key) ^ purpose));
}

// Tunables: read once from the environment (TK_*), changeable at run time through
// tk_debug_set_tunable (benchmarks and tests only; the defaults are the measured best).
// Host code reads them once per launch; atomics keep concurrent readers well defined.
struct Config {
  std::atomic<bool> nt_stores;       // TK_STORE=nt: non-temporal 16-byte stores
  std::atomic<uint64_t> max_blocks;  // TK_MAX_BLOCKS: cap on the grid of the streaming fills
  std::atomic<int> unroll;           // TK_UNROLL: 16-byte vectors per lane per tile (1, 2 or 4)
  std::atomic<int> choice_tiles;     // TK_CHOICE_TILES: 4 KiB tiles per choice work-group (1, 2, 4, 8)
  std::atomic<int> exp_tiles;        // TK_EXP_TILES: 4 KiB tiles per exponential work-group (1, 2, 4)
  std::atomic<int> zig_tiles;        // TK_ZIG_TILES: tiles (one 16-byte vector per lane) per table-pass work-group
  std::atomic<bool> zig_fused;       // TK_ZIG_MODE=fused|split: misses finished in the table pass, or in a second kernel
  std::atomic<bool> zig_lds;         // TK_ZIG_TABLE=lds|global: where the table pass gathers the layers
  std::atomic<bool> philox_lds;      // TK_PHILOX=lds|overlap: Philox fills at word offsets 1..3 by the LDS
                                     // tile kernel or the overlapping-wave kernel
  std::atomic<bool> pair_lds;        // TK_PAIRS=lds|wave: Box-Muller pairs at odd starts by the pair tile
                                     // kernel (the next wave's first value through LDS) or each wave alone
  std::atomic<int> lds_pad;           // TK_LDS_PAD: dynamic LDS bytes per work-group of every streaming fill,
                                     // which caps the groups resident on a CU (-1, unset: each fill's default)
  std::atomic<int> zig_lds_pad;       // TK_ZIG_LDS_PAD: the same for the ziggurat table pass
  std::atomic<int> const_work;       // TK_CONST_WORK: dependent integer steps per lane before each store of
                                     // the constant fill (0: none), to sweep the store ceiling's spacing
};
const Config &config();
// The dynamic LDS bytes of a streaming fill's launch: the op's measured default, unless the
// tunable overrides it.
template <class Op>
inline uint32_t lds_pad() {
  const int v = config().lds_pad;
  return v >= 0 ? (uint32_t)v : Op::kLdsPad;
}

// Compute units of the current device (cached per device).
int device_cus(int device);

// Current device, or a negative value with the error recorded.
int current_device(tk_status *st);

constexpr int kMaxDevices = 64;

// Every device allocation of the library goes through these two: they keep the count of
// bytes the library holds (tk_debug_device_bytes) and fail the allocations a test asks to
// fail (tk_debug_fail_allocations) without calling HIP.  device_free(nullptr, ..) does
// nothing; `bytes` is the size the allocation was made with.
hipError_t device_alloc(void **p, size_t bytes);
hipError_t device_free(void *p, size_t bytes);

}  // namespace tk
