// api_kernels.hip -- test kernels written against include/tk_device_api.h the way a user's
// kernel fuses draws into the statement that uses them (Phobos stdlib, "Random numbers":
// the dropout_rows example, counter = flat index in the whole tensor).  Test
// infrastructure: the GPU tests compare these kernels with the library's fills and with
// the oracle.  Built by tests/build_api_kernels.py into tests/libtk_api_kernels.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tk_device_api.h"

namespace {

constexpr uint32_t kThreads = 256;

__global__ void k_uniform_f32(uint32_t hk, uint32_t c0, uint32_t n, float *out) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = tk_uniform_f32(hk, c0 + i);
}

__global__ void k_uniform_f64(uint32_t hk, uint32_t i0, uint32_t n, double *out) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = tk_uniform_f64(hk, i0 + i);
}

__global__ void k_randn_f32(uint32_t hk, uint32_t c0, uint32_t n, float *out) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = tk_randn_f32(hk, c0 + i);
}

__global__ void k_randn2_f32(uint32_t hk, uint32_t c0, uint32_t npairs, float *out) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < npairs) tk_randn2_f32(hk, c0 + i, &out[2 * i], &out[2 * i + 1]);
}

// A work-group of 256 lanes covers R rows of the [rows, 256] tensor, one column per lane.
template <int R>
__global__ void k_dropout_rows(const float *x, float *y, uint32_t rows, float p, uint32_t hk) {
  const float q = 1.0f - p;
  const uint32_t col = threadIdx.x;
  for (int j = 0; j < R; ++j) {
    const uint32_t row = blockIdx.x * R + j;
    if (row >= rows) break;
    const uint32_t c = row * 256u + col;
    y[c] = tk_dropout_apply_f32(x[c], p, q, hk, c);
  }
}

uint32_t blocks(uint64_t n, uint64_t per) { return (uint32_t)((n + per - 1) / per); }

}  // namespace

// Launchers: plain device pointers, n below 2^31, hipError_t of the launch.
extern "C" {

int tkt_uniform_f32(uint32_t key, uint32_t c0, uint32_t n, float *out, hipStream_t s) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_uniform_f32, dim3(blocks(n, kThreads)), dim3(kThreads), 0, s, tk_key_hash(key), c0, n, out);
  return (int)hipGetLastError();
}

int tkt_uniform_f64(uint32_t key, uint32_t i0, uint32_t n, double *out, hipStream_t s) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_uniform_f64, dim3(blocks(n, kThreads)), dim3(kThreads), 0, s, tk_key_hash(key), i0, n, out);
  return (int)hipGetLastError();
}

int tkt_randn_f32(uint32_t key, uint32_t c0, uint32_t n, float *out, hipStream_t s) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_randn_f32, dim3(blocks(n, kThreads)), dim3(kThreads), 0, s, tk_key_hash(key), c0, n, out);
  return (int)hipGetLastError();
}

int tkt_randn2_f32(uint32_t key, uint32_t c0, uint32_t npairs, float *out, hipStream_t s) {
  if (npairs == 0) return 0;
  hipLaunchKernelGGL(k_randn2_f32, dim3(blocks(npairs, kThreads)), dim3(kThreads), 0, s, tk_key_hash(key), c0,
                     npairs, out);
  return (int)hipGetLastError();
}

// x, y: [rows, 256] f32, rows <= 2^24 (flat counters below 2^32).
int tkt_dropout_rows(uint32_t key, uint32_t rows, float p, const float *x, float *y, hipStream_t s) {
  if (rows == 0) return 0;
  if (rows > (1u << 24)) return (int)hipErrorInvalidValue;
  constexpr int R = 16;
  hipLaunchKernelGGL(k_dropout_rows<R>, dim3(blocks(rows, R)), dim3(256), 0, s, x, y, rows, p, tk_key_hash(key));
  return (int)hipGetLastError();
}

}  // extern "C"
