/*
 * A plain C program using libtk through include/tk.h alone: no C++, no Python, no torch.
 * It fills device buffers on one stream, copies them back and compares them with the C
 * oracle (test infrastructure), and checks the status of calls the header says are
 * refused.  Exit status 0 when everything matches; it prints the first mismatch otherwise.
 *
 * Built by tests/build_c_consumer.py (gcc, linked against bulk_fills_amd/libtk.so and
 * oracle/liboracle.so); run on a GPU by tests/test_c_abi_consumer.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tk.h"
#include "oracle.h"

#define N ((uint64_t)(1u << 18) + 7u)

static int failures = 0;

#define HIP_OK(call)                                                     \
  do {                                                                   \
    hipError_t e_ = (call);                                              \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s:%d: %s -> hip error %d\n", __FILE__, __LINE__, \
              #call, (int)e_);                                           \
      exit(2);                                                           \
    }                                                                    \
  } while (0)

static void expect_status(tk_status got, tk_status want, const char *what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, (int)got, tk_status_string(got), (int)want);
    ++failures;
  }
}

static void expect_bytes(const void *got, const void *want, size_t bytes, size_t elem, const char *what) {
  const unsigned char *g = (const unsigned char *)got, *w = (const unsigned char *)want;
  for (size_t i = 0; i < bytes; i += elem) {
    if (memcmp(g + i, w + i, elem) != 0) {
      fprintf(stderr, "%s: first mismatch at element %zu\n", what, i / elem);
      ++failures;
      return;
    }
  }
}

int main(void) {
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void *dev = NULL;
  HIP_OK(hipMalloc(&dev, N * 8 + 16));
  unsigned char *host = (unsigned char *)malloc(N * 8 + 16);
  unsigned char *want = (unsigned char *)malloc(N * 8 + 16);
  if (!host || !want) return 2;

  /* u32, start 3, from a 4-byte-misaligned device address (head and tail elements) */
  expect_status(tk_fill_u32(1, 3, N, (uint32_t *)((char *)dev + 4), stream), TK_OK, "tk_fill_u32");
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(host, (char *)dev + 4, N * 4, hipMemcpyDeviceToHost));
  if (orc_fill_u32(1, 3, N, NULL, (uint32_t *)want) != 0) return 2;
  expect_bytes(host, want, N * 4, 4, "tk_fill_u32");

  /* u64_below(1000), start 5 */
  expect_status(tk_fill_u64_below(2, 5, N, 1000, (uint64_t *)dev, stream), TK_OK, "tk_fill_u64_below");
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(host, dev, N * 8, hipMemcpyDeviceToHost));
  if (orc_fill_u64_below(2, 5, N, NULL, 1000, (uint64_t *)want) != 0) return 2;
  expect_bytes(host, want, N * 8, 8, "tk_fill_u64_below");

  /* f64 normal (ziggurat), start 1: fast-path and wedge values bit-exact, tail 1e-12 */
  expect_status(tk_fill_normal_f64(3, 1, N, (double *)dev, stream), TK_OK, "tk_fill_normal_f64");
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(host, dev, N * 8, hipMemcpyDeviceToHost));
  uint8_t *path = (uint8_t *)malloc(N);
  if (!path || orc_fill_normal_f64(3, 1, N, NULL, (double *)want, path) != 0) return 2;
  for (uint64_t i = 0; i < N; ++i) {
    const double g = ((const double *)host)[i], w = ((const double *)want)[i];
    const int ok = path[i] == 2 ? fabs(g - w) <= 1e-12 * fabs(w) : memcmp(&g, &w, 8) == 0;
    if (!ok) {
      fprintf(stderr, "tk_fill_normal_f64: mismatch at %llu (path %d): %.17g vs %.17g\n",
              (unsigned long long)i, path[i], g, w);
      ++failures;
      break;
    }
  }

  /* choice through an alias table of 1000 Zipf(1.1) weights */
  double weights[1000];
  uint32_t q[1000], alias[1000];
  uint64_t mass[1000];
  for (int j = 0; j < 1000; ++j) weights[j] = pow((double)(j + 1), -1.1);
  tk_alias *table = NULL;
  expect_status(tk_alias_create(weights, 1000, &table), TK_OK, "tk_alias_create");
  if (table) {
    expect_status(tk_fill_choice_u32(4, 0, N, table, (uint32_t *)dev, stream), TK_OK, "tk_fill_choice_u32");
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(host, dev, N * 4, hipMemcpyDeviceToHost));
    if (orc_alias_build(weights, 1000, q, alias, mass) != 0) return 2;
    if (orc_fill_choice_u32(4, 0, N, NULL, q, alias, 1000, (uint32_t *)want) != 0) return 2;
    expect_bytes(host, want, N * 4, 4, "tk_fill_choice_u32");
    expect_status(tk_alias_destroy(table), TK_OK, "tk_alias_destroy");
  }

  /* refused calls enqueue nothing and say why */
  expect_status(tk_fill_u32(1, 0, 16, NULL, stream), TK_EINVAL, "NULL output");
  expect_status(tk_fill_u32(1, 0, 16, (uint32_t *)((char *)dev + 1), stream), TK_EINVAL, "misaligned output");
  expect_status(tk_fill_u32(1, 0xFFFFFFF0ull, 32, (uint32_t *)dev, stream), TK_ERANGE, "past the counter space");
  expect_status(tk_fill_u32_below(1, 0, 16, 0, (uint32_t *)dev, stream), TK_EINVAL, "bound 0");
  expect_status(tk_fill_u32(1, 0, 0, NULL, stream), TK_OK, "n = 0");
  expect_status(tk_dropout_f32(1, 0, 16, 1.0f, (const float *)dev, (float *)dev, NULL, stream), TK_EINVAL, "p = 1");

  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipFree(dev));
  HIP_OK(hipStreamDestroy(stream));
  free(path);
  free(host);
  free(want);
  printf("c_abi_consumer: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
