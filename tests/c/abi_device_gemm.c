/* Device use of libmfl.so from plain C99 through include/mfl.h and the HIP
 * runtime's C API: fp32 operands are rounded to bf16 on the device
 * (quantize_fp32), multiplied with gemm_tile_mma (A row-major, B column-major,
 * padded leading dimensions, C with a padding column that must stay untouched),
 * and sampled entries of C are compared with a double-precision dot product of
 * the rounded values read back from the device.  Two sizes: whole 256 x 256
 * tiles, and a ragged one.  Exit status 0 on success; the first failure is
 * printed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mfl.h"

#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static float uniform_pm1(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((double)(lcg >> 11) / (double)(1ull << 53) * 2.0 - 1.0);
}
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Fills rows x ld storage (the first `cols` of each row valid, the rest NaN),
 * rounds it to bf16 on the device and returns both copies. */
static int make_operand(int64_t rows, int64_t cols, int64_t ld, void** dev16, uint16_t** host16) {
  const int64_t n = rows * ld;
  float* h = (float*)malloc((size_t)n * sizeof(float));
  CHECK(h != NULL);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < ld; ++c) h[r * ld + c] = c < cols ? uniform_pm1() : NAN;
  float* d32 = NULL;
  CHECK(hipMalloc((void**)&d32, (size_t)n * sizeof(float)) == hipSuccess);
  CHECK(hipMalloc(dev16, (size_t)n * sizeof(uint16_t)) == hipSuccess);
  CHECK(hipMemcpy(d32, h, (size_t)n * sizeof(float), hipMemcpyHostToDevice) == hipSuccess);
  CHECK(quantize_fp32(MFL_BF16, d32, *dev16, n, NULL) == MFL_OK);
  *host16 = (uint16_t*)malloc((size_t)n * sizeof(uint16_t));
  CHECK(*host16 != NULL);
  CHECK(hipMemcpy(*host16, *dev16, (size_t)n * sizeof(uint16_t), hipMemcpyDeviceToHost) == hipSuccess);
  CHECK(hipFree(d32) == hipSuccess);
  free(h);
  return 0;
}

static int run(int64_t m, int64_t n, int64_t k) {
  const int64_t ld = k + 64, ldc = n + 1;
  void *da = NULL, *db = NULL;
  uint16_t *ha = NULL, *hb = NULL;
  if (make_operand(m, k, ld, &da, &ha) || make_operand(n, k, ld, &db, &hb)) return 1;
  float* dc = NULL;
  const size_t cbytes = (size_t)(m * ldc) * sizeof(float);
  CHECK(hipMalloc((void**)&dc, cbytes) == hipSuccess);
  float* hc = (float*)malloc(cbytes);
  CHECK(hc != NULL);
  for (int64_t i = 0; i < m * ldc; ++i) hc[i] = 12345.0f;
  CHECK(hipMemcpy(dc, hc, cbytes, hipMemcpyHostToDevice) == hipSuccess);
  CHECK(gemm_tile_mma(MFL_BF16, m, n, k, da, ld, MFL_ROW_MAJOR, db, ld, MFL_COL_MAJOR, dc, ldc, 0, NULL) == MFL_OK);
  CHECK(hipDeviceSynchronize() == hipSuccess);
  CHECK(hipMemcpy(hc, dc, cbytes, hipMemcpyDeviceToHost) == hipSuccess);
  double err2 = 0.0, ref2 = 0.0;
  for (int s = 0; s < 4096; ++s) {
    const int64_t i = (int64_t)(s * 7919) % m, j = (int64_t)(s * 104729 + s / 7) % n;
    double ref = 0.0;
    for (int64_t t = 0; t < k; ++t) ref += bf16_value(ha[i * ld + t]) * bf16_value(hb[j * ld + t]);
    const double d = (double)hc[i * ldc + j] - ref;
    err2 += d * d;
    ref2 += ref * ref;
  }
  for (int64_t i = 0; i < m; ++i) CHECK(hc[i * ldc + n] == 12345.0f); /* padding column untouched */
  const double rel = sqrt(err2 / ref2);
  printf("abi_device_gemm: %lld x %lld x %lld bf16, sampled normwise error %.3e\n", (long long)m, (long long)n,
         (long long)k, rel);
  CHECK(rel <= 1e-5);
  CHECK(hipFree(da) == hipSuccess && hipFree(db) == hipSuccess && hipFree(dc) == hipSuccess);
  free(ha);
  free(hb);
  free(hc);
  return 0;
}

int main(void) {
  int count = 0;
  CHECK(hipGetDeviceCount(&count) == hipSuccess && count > 0);
  if (run(1024, 768, 512) || run(1000, 520, 200)) return 1;
  printf("abi_device_gemm: ok\n");
  return 0;
}
