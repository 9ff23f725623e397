/* A C-only client of the library: device buffers from hipMalloc, plans from
 * cbd_plan, runs through cbd_run on the default stream, results copied back
 * and compared bit for bit with the oracle on integer-valued operands (every
 * partial sum is an integer below 2^24, so fp32 accumulation is exact and
 * the expected value is the oracle's result rounded once to the output
 * dtype).  No torch and no Python anywhere: the library interface as a
 * plain client sees it.  Exit status 0 and "CLIENT OK" on success.
 *
 * Test infrastructure: links the oracle (oracle/cbd_oracle.c) only to
 * compute the expected values. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "cbd.h"

int cbd_oracle_out_hw(const int64_t* p, int64_t* ho_wo);
int cbd_oracle_bwd_data(const int64_t* p, const double* dy, const double* w, double* dx);
void cbd_oracle_round_f32(int64_t n, const double* in, float* out);
void cbd_oracle_round_bf16(int64_t n, const float* in, uint16_t* out);

#define HIPCHECK(x)                                                        \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));      \
      exit(2);                                                             \
    }                                                                      \
  } while (0)

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static int small_int(void) {
  rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
  return (int)(rs % 5) - 2;
}

/* One problem: returns 0 if the GPU result is bit-exact. */
static int run_case(const char* name, cbd_problem pr, int expect_kernel) {
  cbd_plan_t* plan = NULL;
  cbd_status st = cbd_plan(&pr, &plan);
  if (st != CBD_OK) {
    fprintf(stderr, "%s: cbd_plan: %s (%s)\n", name, cbd_status_string(st), cbd_last_error());
    return 1;
  }
  cbd_plan_info_t info;
  if (cbd_plan_info(plan, &info) != CBD_OK) return 1;
  if (expect_kernel >= 0 && info.kernel != expect_kernel) {
    fprintf(stderr, "%s: kernel %d, expected %d\n", name, info.kernel, expect_kernel);
    return 1;
  }
  const int64_t cg = pr.c / pr.g;
  const int64_t nx = pr.n * pr.c * pr.hi * pr.wi, ny = pr.n * pr.k * info.ho * info.wo;
  const int64_t nw = pr.k * cg * pr.y * pr.x;
  const size_t es = pr.dtype == CBD_F32 ? 4 : 2;
  double* dy = malloc(sizeof(double) * ny);
  double* w = malloc(sizeof(double) * nw);
  double* ref = malloc(sizeof(double) * nx);
  float* ref32 = malloc(sizeof(float) * nx);
  uint16_t* ref16 = malloc(sizeof(uint16_t) * nx);
  void* hdy = malloc(es * ny);
  void* hw = malloc(es * nw);
  void* hdx = malloc(es * nx);
  for (int64_t i = 0; i < ny; i++) dy[i] = small_int();
  for (int64_t i = 0; i < nw; i++) w[i] = small_int();
  /* small integers are exact in f32 and bf16: bf16 bits = top half of the f32 bits */
  for (int64_t i = 0; i < ny; i++) {
    float f = (float)dy[i];
    uint32_t u;
    memcpy(&u, &f, 4);
    if (es == 4) ((float*)hdy)[i] = f; else ((uint16_t*)hdy)[i] = (uint16_t)(u >> 16);
  }
  for (int64_t i = 0; i < nw; i++) {
    float f = (float)w[i];
    uint32_t u;
    memcpy(&u, &f, 4);
    if (es == 4) ((float*)hw)[i] = f; else ((uint16_t*)hw)[i] = (uint16_t)(u >> 16);
  }
  int64_t pv[15] = {pr.n, pr.g, pr.c, pr.k, pr.hi, pr.wi, pr.y, pr.x, pr.stride_h, pr.stride_w,
                    pr.pad_h, pr.pad_w, pr.dil_h, pr.dil_w, pr.layout};
  if (cbd_oracle_bwd_data(pv, dy, w, ref)) return 1;
  cbd_oracle_round_f32(nx, ref, ref32);
  cbd_oracle_round_bf16(nx, ref32, ref16);

  void *ddy, *dw, *ddx;
  HIPCHECK(hipMalloc(&ddy, es * ny));
  HIPCHECK(hipMalloc(&dw, es * nw));
  HIPCHECK(hipMalloc(&ddx, es * nx));
  HIPCHECK(hipMemcpy(ddy, hdy, es * ny, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dw, hw, es * nw, hipMemcpyHostToDevice));
  HIPCHECK(hipMemset(ddx, 0xff, es * nx)); /* NaN pattern: every element must be written */
  /* argument errors come back as status codes */
  if (cbd_run(plan, NULL, dw, ddx, NULL) != CBD_ERR_INVALID_ARG) {
    fprintf(stderr, "%s: NULL dy not refused\n", name);
    return 1;
  }
  st = cbd_run(plan, ddy, dw, ddx, NULL);
  if (st != CBD_OK) {
    fprintf(stderr, "%s: cbd_run: %s (%s)\n", name, cbd_status_string(st), cbd_last_error());
    return 1;
  }
  HIPCHECK(hipDeviceSynchronize());
  HIPCHECK(hipMemcpy(hdx, ddx, es * nx, hipMemcpyDeviceToHost));
  int64_t bad = 0;
  for (int64_t i = 0; i < nx; i++) {
    if (es == 4) {
      uint32_t a, b;
      memcpy(&a, &((float*)hdx)[i], 4);
      memcpy(&b, &ref32[i], 4);
      bad += a != b;
    } else {
      bad += ((uint16_t*)hdx)[i] != ref16[i];
    }
  }
  printf("%s: kernel %d, %d sub-GEMMs, %d zero regions, %lld elements, %lld mismatches\n", name,
         info.kernel, info.num_subgemms, info.num_zero_regions, (long long)nx, (long long)bad);
  HIPCHECK(hipFree(ddy));
  HIPCHECK(hipFree(dw));
  HIPCHECK(hipFree(ddx));
  cbd_plan_destroy(plan);
  free(dy); free(w); free(ref); free(ref32); free(ref16); free(hdy); free(hw); free(hdx);
  return bad != 0;
}

static cbd_problem mk(int64_t n, int64_t g, int64_t c, int64_t k, int64_t hi, int64_t wi, int64_t y,
                      int64_t x, int s_h, int s_w, int p_h, int p_w, int layout, int dtype) {
  cbd_problem p;
  memset(&p, 0, sizeof(p));
  p.n = n; p.g = g; p.c = c; p.k = k; p.hi = hi; p.wi = wi; p.y = y; p.x = x;
  p.stride_h = s_h; p.stride_w = s_w; p.pad_h = p_h; p.pad_w = p_w; p.dil_h = 1; p.dil_w = 1;
  p.layout = layout; p.dtype = dtype;
  return p;
}

int main(void) {
  int fails = 0;
  cbd_plan_destroy(NULL);
  if (cbd_plan(NULL, NULL) != CBD_ERR_INVALID_ARG) fails++;
  /* fp32 NCHW stride 2 3x3 (generic family) */
  fails += run_case("f32-nchw-3x3-s2", mk(2, 1, 24, 20, 15, 13, 3, 3, 2, 2, 1, 1, CBD_LAYOUT_NCHW, CBD_F32),
                    CBD_KERNEL_GENERIC);
  /* fp32 NCHW 1x1 stride 2 (three zero phases, folded zero-fill) */
  fails += run_case("f32-nchw-1x1-s2", mk(2, 1, 16, 16, 14, 14, 1, 1, 2, 2, 0, 0, CBD_LAYOUT_NCHW, CBD_F32),
                    CBD_KERNEL_GENERIC);
  /* fp32 NHWC 3x3 stride 2 with 3 groups (generic family) */
  fails += run_case("f32-nhwc-grouped-generic", mk(2, 3, 24, 18, 11, 9, 3, 3, 2, 2, 1, 1, CBD_LAYOUT_NHWC, CBD_F32),
                    CBD_KERNEL_GENERIC);
  /* bf16 NHWC 1x2 stride (1,2): the large-tile kernel */
  fails += run_case("bf16-nhwc-1x2", mk(2, 1, 256, 64, 1, 64, 1, 2, 1, 2, 0, 0, CBD_LAYOUT_NHWC, CBD_BF16),
                    CBD_KERNEL_NHWC_BF16);
  /* bf16 NHWC grouped, 32 groups of 4 channels, 3x3 stride 2 */
  fails += run_case("bf16-grouped", mk(2, 32, 128, 128, 12, 12, 3, 3, 2, 2, 1, 1, CBD_LAYOUT_NHWC, CBD_BF16),
                    CBD_KERNEL_GROUPED);
  if (fails) {
    printf("CLIENT FAILED (%d)\n", fails);
    return 1;
  }
  printf("CLIENT OK\n");
  return 0;
}
