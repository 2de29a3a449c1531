// Philox4x32-10 words from rocRAND's engine (ROCm's random-number library, its header-only
// implementation, run on the host): an implementation independent of the oracle's, against
// which the tests pin the oracle's Philox word source.
//
// rocrand_init(seed, subsequence, offset) starts the engine at key (lo32 seed, hi32 seed),
// counter words 0-1 = offset / 4 and words 2-3 = subsequence, lane offset % 4; every call
// of rocrand() then returns the next word of that stream.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <stdint.h>

extern "C" void rocrand_ref_philox_words(uint64_t seed, uint64_t subsequence, uint64_t offset, uint64_t n,
                                         uint32_t *out) {
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, subsequence, offset, &st);
  for (uint64_t i = 0; i < n; ++i) out[i] = rocrand(&st);
}
