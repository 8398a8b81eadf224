/*
 * A torch-free consumer of the C ABI (include/adaln.h) on the GPU: plain C11,
 * HIP runtime calls for memory and a stream, and the library's entry points.
 * It checks properties that hold for any correct implementation rather than
 * element values (those are the Python parity tests' job against the fp64
 * oracle):
 *   - with scale = shift = 0 every output row has mean 0 and mean square
 *     var / (var + eps)  (LayerNorm without affine);
 *   - every dx row sums to 0;
 *   - dshift[b, d] is the sum over the sample's rows of dy[r, d]  (computed
 *     here in double from the same inputs);
 *   - adaln_bwd_f32sums returns the same dx and the same sums as adaln_bwd
 *     for fp32 I/O, bit for bit; a second adaln_bwd call repeats the first
 *     bit for bit;
 *   - the documented errors come back for a null pointer and a short workspace.
 * Exit status 0 and a final "OK" line on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "adaln.h"

#define CHECK_HIP(call)                                                         \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 2;                                                                 \
    }                                                                           \
  } while (0)

#define EXPECT(cond, ...)              \
  do {                                 \
    if (!(cond)) {                     \
      fprintf(stderr, "FAIL: ");       \
      fprintf(stderr, __VA_ARGS__);    \
      fprintf(stderr, "\n");           \
      return 1;                        \
    }                                  \
  } while (0)

/* splitmix64: a fixed, seeded stream of test values */
static uint64_t mix_state = 0x9E3779B97F4A7C15ull;
static double next_unit(void) {
  uint64_t z = (mix_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0; /* [-1, 1) */
}

int main(void) {
  const int64_t B = 3, N = 700, D = 1152, R = B * N;
  const float eps = 1e-6f;
  const size_t rows_bytes = (size_t)(R * D) * sizeof(float), mod_bytes = (size_t)(B * D) * sizeof(float);
  float *hx = malloc(rows_bytes), *hdy = malloc(rows_bytes), *hy = malloc(rows_bytes),
        *hdx = malloc(rows_bytes), *hdx2 = malloc(rows_bytes), *hzero = calloc((size_t)(B * D), sizeof(float)),
        *hdsh = malloc(mod_bytes), *hdsc = malloc(mod_bytes), *hdsh2 = malloc(mod_bytes),
        *hdsc2 = malloc(mod_bytes), *hdsh3 = malloc(mod_bytes), *hdx3 = malloc(rows_bytes);
  if (!hx || !hdy || !hy || !hdx || !hdx2 || !hzero || !hdsh || !hdsc || !hdsh2 || !hdsc2 || !hdsh3 || !hdx3) return 2;
  for (int64_t i = 0; i < R * D; ++i) {
    const int64_t r = i / D;
    hx[i] = (float)(next_unit() * 1.7 + 0.25 * (double)(r % 7));   /* rows off zero mean */
    hdy[i] = (float)(next_unit() * 1e-2);
  }

  hipStream_t st;
  CHECK_HIP(hipStreamCreate(&st));
  void *x, *dy, *y, *dx, *sh, *sc, *dsh, *dsc, *ws;
  float *mean, *rstd;
  CHECK_HIP(hipMalloc(&x, rows_bytes));
  CHECK_HIP(hipMalloc(&dy, rows_bytes));
  CHECK_HIP(hipMalloc(&y, rows_bytes));
  CHECK_HIP(hipMalloc(&dx, rows_bytes));
  CHECK_HIP(hipMalloc(&sh, mod_bytes));
  CHECK_HIP(hipMalloc(&sc, mod_bytes));
  CHECK_HIP(hipMalloc(&dsh, mod_bytes));
  CHECK_HIP(hipMalloc(&dsc, mod_bytes));
  CHECK_HIP(hipMalloc((void**)&mean, (size_t)R * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&rstd, (size_t)R * sizeof(float)));
  const size_t wsb = adaln_bwd_workspace_size(B, R, D, ADALN_F32);
  EXPECT(wsb > 0, "workspace size query returned 0");
  CHECK_HIP(hipMalloc(&ws, wsb));
  CHECK_HIP(hipMemcpy(x, hx, rows_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dy, hdy, rows_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(sh, hzero, mod_bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(sc, hzero, mod_bytes, hipMemcpyHostToDevice));

  EXPECT(adaln_abi_version() == ADALN_ABI_VERSION, "ABI version %d, header %d", adaln_abi_version(), ADALN_ABI_VERSION);
  adaln_status_t s = adaln_fwd(x, sh, sc, eps, B, N, D, ADALN_F32, st, y, mean, rstd);
  EXPECT(s == ADALN_OK, "adaln_fwd: %s", adaln_status_str(s));
  s = adaln_bwd(dy, x, sc, mean, rstd, B, N, D, ADALN_F32, ws, wsb, st, dx, dsc, dsh);
  EXPECT(s == ADALN_OK, "adaln_bwd: %s", adaln_status_str(s));
  CHECK_HIP(hipStreamSynchronize(st));
  CHECK_HIP(hipMemcpy(hy, y, rows_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdx, dx, rows_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdsh, dsh, mod_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdsc, dsc, mod_bytes, hipMemcpyDeviceToHost));

  for (int64_t r = 0; r < R; ++r) {
    double m = 0.0, q = 0.0, v = 0.0, sdx = 0.0, adx = 0.0, mx = 0.0;
    for (int64_t d = 0; d < D; ++d) mx += hx[r * D + d];
    mx /= (double)D;
    for (int64_t d = 0; d < D; ++d) {
      const double yy = hy[r * D + d], t = hx[r * D + d] - mx;
      m += yy; q += yy * yy; v += t * t;
      sdx += hdx[r * D + d]; adx += fabs(hdx[r * D + d]);
    }
    m /= (double)D; q /= (double)D; v /= (double)D;
    const double want_q = v / (v + (double)eps);
    EXPECT(fabs(m) < 1e-5, "row %lld: mean of y %g", (long long)r, m);
    EXPECT(fabs(q - want_q) < 1e-4, "row %lld: mean square of y %g, want %g", (long long)r, q, want_q);
    EXPECT(fabs(sdx) <= 1e-4 * adx + 1e-12, "row %lld: sum of dx %g (sum |dx| %g)", (long long)r, sdx, adx);
  }
  for (int64_t b = 0; b < B; ++b)
    for (int64_t d = 0; d < D; ++d) {
      double want = 0.0, mag = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        want += hdy[(b * N + n) * D + d];
        mag += fabs(hdy[(b * N + n) * D + d]);
      }
      const double got = hdsh[b * D + d];
      EXPECT(fabs(got - want) <= 1e-5 * mag, "dshift[%lld,%lld] = %.9g, want %.9g", (long long)b, (long long)d, got, want);
    }

  /* fp32 sums entry point: same dx and sums, bit for bit, for fp32 I/O */
  s = adaln_bwd_f32sums(dy, x, sc, mean, rstd, B, N, D, ADALN_F32, ws, wsb, st, dx, (float*)dsc, (float*)dsh);
  EXPECT(s == ADALN_OK, "adaln_bwd_f32sums: %s", adaln_status_str(s));
  CHECK_HIP(hipStreamSynchronize(st));
  CHECK_HIP(hipMemcpy(hdx2, dx, rows_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdsh2, dsh, mod_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdsc2, dsc, mod_bytes, hipMemcpyDeviceToHost));
  EXPECT(memcmp(hdx, hdx2, rows_bytes) == 0, "adaln_bwd_f32sums dx differs from adaln_bwd's");
  EXPECT(memcmp(hdsh, hdsh2, mod_bytes) == 0 && memcmp(hdsc, hdsc2, mod_bytes) == 0,
         "adaln_bwd_f32sums sums differ from adaln_bwd's");
  /* run to run */
  s = adaln_bwd(dy, x, sc, mean, rstd, B, N, D, ADALN_F32, ws, wsb, st, dx, dsc, dsh);
  EXPECT(s == ADALN_OK, "adaln_bwd (again): %s", adaln_status_str(s));
  CHECK_HIP(hipStreamSynchronize(st));
  CHECK_HIP(hipMemcpy(hdx3, dx, rows_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hdsh3, dsh, mod_bytes, hipMemcpyDeviceToHost));
  EXPECT(memcmp(hdx, hdx3, rows_bytes) == 0 && memcmp(hdsh, hdsh3, mod_bytes) == 0, "a second call differs");

  /* documented errors, nothing launched */
  s = adaln_bwd(dy, x, sc, mean, rstd, B, N, D, ADALN_F32, ws, 64, st, dx, dsc, dsh);
  EXPECT(s == ADALN_ERR_WORKSPACE_TOO_SMALL, "short workspace: %s", adaln_status_str(s));
  s = adaln_fwd(NULL, sh, sc, eps, B, N, D, ADALN_F32, st, y, mean, rstd);
  EXPECT(s == ADALN_ERR_INVALID_ARG, "null x: %s", adaln_status_str(s));

  CHECK_HIP(hipStreamSynchronize(st));
  void* bufs[] = {x, dy, y, dx, sh, sc, dsh, dsc, mean, rstd, ws};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) CHECK_HIP(hipFree(bufs[i]));
  CHECK_HIP(hipStreamDestroy(st));
  free(hx); free(hdy); free(hy); free(hdx); free(hdx2); free(hzero); free(hdsh); free(hdsc);
  free(hdsh2); free(hdsc2); free(hdsh3); free(hdx3);
  printf("OK: %lld rows x %lld features, %d samples\n", (long long)R, (long long)D, (int)B);
  return 0;
}
