/*
 * A plain C consumer of the library: device buffers from hipMalloc, one
 * flce_fwd_bwd call and one flce_fwd call on the null stream, and an argument
 * error.  Inputs come from a 32-bit linear congruential generator whose values
 * k / 64 (k in [-64, 64]) are exact in fp32, so the test that runs this program
 * rebuilds the same inputs in Python and checks the printed results against
 * the oracle.  Output: one "name value..." line per quantity.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "flce.h"

static uint32_t g_state;

static uint32_t next_u32(void) {
  g_state = g_state * 1664525u + 1013904223u;
  return g_state;
}

/* one of the 129 values k / 64, k in [-64, 64] */
static float next_value(void) { return (float)((int)((next_u32() >> 16) % 129u) - 64) / 64.0f; }

#define CHECK_HIP(x)                                                  \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); \
      return 2;                                                       \
    }                                                                 \
  } while (0)

static void print_array(const char* name, const float* x, int64_t count) {
  printf("%s", name);
  for (int64_t i = 0; i < count; ++i) printf(" %.9e", (double)x[i]);
  printf("\n");
}

int main(void) {
  const int64_t n = 24, d = 16, v = 40;
  float h[24 * 16], w[40 * 16], lse[24], dh[24 * 16], dw[40 * 16], loss, loss_fwd, lse_fwd[24];
  int64_t labels[24];
  g_state = 12345u;
  for (int64_t i = 0; i < n * d; ++i) h[i] = next_value();
  for (int64_t i = 0; i < v * d; ++i) w[i] = next_value() * 0.5f;
  for (int64_t i = 0; i < n; ++i) labels[i] = (i % 5 == 4) ? -100 : (int64_t)(next_u32() % (uint32_t)v);

  void *dh_d, *dw_d, *h_d, *w_d;
  float *lse_d, *loss_d, *lse2_d, *loss2_d;
  int64_t* y_d;
  CHECK_HIP(hipMalloc(&h_d, sizeof(h)));
  CHECK_HIP(hipMalloc(&w_d, sizeof(w)));
  CHECK_HIP(hipMalloc((void**)&y_d, sizeof(labels)));
  CHECK_HIP(hipMalloc(&dh_d, sizeof(dh)));
  CHECK_HIP(hipMalloc(&dw_d, sizeof(dw)));
  CHECK_HIP(hipMalloc((void**)&lse_d, sizeof(lse)));
  CHECK_HIP(hipMalloc((void**)&loss_d, sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&lse2_d, sizeof(lse)));
  CHECK_HIP(hipMalloc((void**)&loss2_d, sizeof(float)));
  CHECK_HIP(hipMemcpy(h_d, h, sizeof(h), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(w_d, w, sizeof(w), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(y_d, labels, sizeof(labels), hipMemcpyHostToDevice));

  const int st = flce_fwd_bwd(h_d, w_d, y_d, n, d, v, FLCE_F32, -100, FLCE_MEAN, loss_d, lse_d, dh_d, dw_d, 0);
  const int st_fwd = flce_fwd(h_d, w_d, y_d, n, d, v, FLCE_F32, -100, FLCE_MEAN, loss2_d, lse2_d, 0);
  const int st_bad = flce_fwd_bwd(h_d, w_d, y_d, 0, d, v, FLCE_F32, -100, FLCE_MEAN, loss_d, lse_d, dh_d, dw_d, 0);
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(&loss, loss_d, sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse, lse_d, sizeof(lse), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dh, dh_d, sizeof(dh), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dw, dw_d, sizeof(dw), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(&loss_fwd, loss2_d, sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse_fwd, lse2_d, sizeof(lse), hipMemcpyDeviceToHost));

  printf("status %d %d %d\n", st, st_fwd, st_bad);
  printf("error %s\n", flce_strerror(st_bad));
  print_array("loss", &loss, 1);
  print_array("lse", lse, n);
  print_array("loss_fwd", &loss_fwd, 1);
  print_array("lse_fwd", lse_fwd, n);
  print_array("dh", dh, n * d);
  print_array("dw", dw, v * d);
  hipFree(h_d); hipFree(w_d); hipFree(y_d); hipFree(dh_d); hipFree(dw_d);
  hipFree(lse_d); hipFree(loss_d); hipFree(lse2_d); hipFree(loss2_d);
  return 0;
}
