// Host-side argument validation of every C-ABI entry point (include/nvfp4.h), built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code and driven by
// tests/test_abi_sanitize.py on a machine without a GPU.
//
// Every call made here either fails validation (null pointer, bad shape, misaligned
// pointer, bad scale or element code, short workspace, a problem beyond the static
// scratch), is empty (M or N zero), or is a host-only query (plans, workspace sizes,
// status strings, the global scale from an amax), so no call reaches a kernel launch.
// The pointers are host addresses; they are never dereferenced by the library.
// The shape fuzz feeds the plan and size queries with extreme values (negative, zero,
// powers of two around the 32- and 64-bit limits) so that the sanitizers see every
// overflow check; it also checks that each entry point rejects exactly the shapes its
// plan query rejects.
//
// Prints "checks <n> failures <f>" and exits nonzero on a failure (the sanitizers abort
// on their own findings).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <vector>

#include "nvfp4.h"

namespace {

long g_checks = 0, g_fail = 0;

void expect(int got, int want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    ++g_fail;
    if (g_fail <= 20) fprintf(stderr, "line %d: %s: status %d, expected %d\n", line, what, got, want);
  }
}
#define EXPECT(expr, want) expect((expr), (want), #expr, __LINE__)

void expect_true(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_fail;
    if (g_fail <= 20) fprintf(stderr, "line %d: %s failed\n", line, what);
  }
}
#define EXPECT_TRUE(expr) expect_true((expr), #expr, __LINE__)

alignas(256) uint8_t g_buf[4096];

constexpr int OK = NVFP4_SUCCESS, VAL = NVFP4_ERROR_INVALID_VALUE, SHAPE = NVFP4_ERROR_INVALID_SHAPE,
              MIS = NVFP4_ERROR_MISALIGNED, WS = NVFP4_ERROR_WORKSPACE, BIG = NVFP4_ERROR_TOO_LARGE;

const float kBadScales[] = {0.0f, -1.0f, NAN, INFINITY, -INFINITY, 0x1p-91f, 0x1p91f, 1e-45f};

}  // namespace

int main() {
  void* p = g_buf;               // 256-byte aligned
  void* m2 = g_buf + 2;          // 2-byte aligned only
  void* m8 = g_buf + 8;          // 8-byte aligned only
  void* st = nullptr;            // stream
  const float gs = 1.0f;
  float* dgs = (float*)(g_buf + 64);

  // ---- version, status strings, host global scale ----
  EXPECT(nvfp4_abi_version(), NVFP4_ABI_VERSION);
  for (int s = -3; s < 20; ++s) EXPECT_TRUE(nvfp4_status_string(s) != nullptr);
  EXPECT_TRUE(nvfp4_global_scale_from_amax(0.0f) == 1.0f);
  EXPECT_TRUE(nvfp4_global_scale_from_amax(2688.0f) == 1.0f);
  EXPECT_TRUE(isnan(nvfp4_global_scale_from_amax(-1.0f)));
  EXPECT_TRUE(isnan(nvfp4_global_scale_from_amax(NAN)));
  EXPECT_TRUE(isnan(nvfp4_global_scale_from_amax(INFINITY)));
  EXPECT_TRUE(nvfp4_global_scale_from_amax(std::numeric_limits<float>::denorm_min()) >= 0.0f);
  EXPECT_TRUE(isfinite(nvfp4_global_scale_from_amax(std::numeric_limits<float>::max())));

  // ---- nvfp4_quantize ----
  EXPECT(nvfp4_quantize(nullptr, 4, 64, gs, p, p, st), VAL);
  EXPECT(nvfp4_quantize(p, 4, 64, gs, nullptr, p, st), VAL);
  EXPECT(nvfp4_quantize(p, 4, 64, gs, p, nullptr, st), VAL);
  for (float b : kBadScales) EXPECT(nvfp4_quantize(p, 4, 64, b, p, p, st), VAL);
  EXPECT(nvfp4_quantize(p, -1, 64, gs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize(p, 4, 0, gs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize(p, 4, 8, gs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize(p, 4, 72, gs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize(p, (int64_t)1 << 40, (int64_t)1 << 40, gs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize(p, INT64_MAX, 16, gs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize(m2, 4, 64, gs, p, p, st), MIS);
  EXPECT(nvfp4_quantize(p, 4, 64, gs, m8, p, st), MIS);
  EXPECT(nvfp4_quantize(p, 4, 64, gs, p, m2, st), MIS);
  EXPECT(nvfp4_quantize(p, 0, 64, gs, p, p, st), OK);

  // ---- nvfp4_gemm and its plan ----
  EXPECT(nvfp4_gemm(nullptr, p, gs, p, p, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm(p, nullptr, gs, p, p, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm(p, p, gs, nullptr, p, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm(p, p, gs, p, nullptr, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, 4, 4, 64, nullptr, st), VAL);
  for (float b : kBadScales) {
    EXPECT(nvfp4_gemm(p, p, b, p, p, gs, 4, 4, 64, p, st), VAL);
    EXPECT(nvfp4_gemm(p, p, gs, p, p, b, 4, 4, 64, p, st), VAL);
  }
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, -4, 4, 64, p, st), SHAPE);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, 4, -4, 64, p, st), SHAPE);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, 4, 4, 40, p, st), SHAPE);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, (int64_t)1 << 31, (int64_t)1 << 31, 64, p, st), SHAPE);
  EXPECT(nvfp4_gemm(m2, p, gs, p, p, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm(p, m2, gs, p, p, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm(p, p, gs, m8, p, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm(p, p, gs, p, m2, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, 4, 4, 64, m8, st), MIS);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, 0, 4, 64, p, st), OK);
  EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, 4, 0, 64, p, st), OK);
  int kind = -1;
  EXPECT(nvfp4_gemm_plan(4, 4, 64, 0, nullptr), VAL);
  EXPECT(nvfp4_gemm_plan(4608, 3072, 3072, 0, &kind), OK);
  EXPECT_TRUE(kind == NVFP4_GEMM_FIT);

  // ---- W4A16 and its plan ----
  EXPECT(nvfp4_gemm_w4a16(nullptr, p, p, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm_w4a16(p, nullptr, p, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm_w4a16(p, p, nullptr, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm_w4a16(p, p, p, gs, 4, 4, 64, nullptr, st), VAL);
  for (float b : kBadScales) EXPECT(nvfp4_gemm_w4a16(p, p, p, b, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm_w4a16(p, p, p, gs, 4, 4, 48, p, st), SHAPE);
  EXPECT(nvfp4_gemm_w4a16(p, p, p, gs, 4, 4, ((int64_t)1 << 22) + 32, p, st), SHAPE);
  EXPECT(nvfp4_gemm_w4a16(m8, p, p, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm_w4a16(p, m8, p, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm_w4a16(p, p, m2, gs, 4, 4, 64, p, st), MIS);
  EXPECT(nvfp4_gemm_w4a16(p, p, p, gs, 4, 4, 64, m8, st), MIS);
  EXPECT(nvfp4_gemm_w4a16(p, p, p, gs, 0, 4, 64, p, st), OK);
  EXPECT(nvfp4_gemm_w4a16_plan(4, 4, 64, 0, nullptr), VAL);
  EXPECT(nvfp4_gemm_w4a16_plan(4608, 3072, 3072, 0, &kind), OK);
  EXPECT_TRUE(kind == NVFP4_W4A16_WIDE);

  // ---- MXFP8 (both element types) ----
  for (int e : {0, 1}) {
    EXPECT(nvfp4_mxfp8_quantize_elem(nullptr, 4, 64, e, p, p, st), VAL);
    EXPECT(nvfp4_mxfp8_quantize_elem(p, 4, 64, e, nullptr, p, st), VAL);
    EXPECT(nvfp4_mxfp8_quantize_elem(p, 4, 64, e, p, nullptr, st), VAL);
    EXPECT(nvfp4_mxfp8_quantize_elem(p, 4, 48, e, p, p, st), SHAPE);
    EXPECT(nvfp4_mxfp8_quantize_elem(p, -4, 64, e, p, p, st), SHAPE);
    EXPECT(nvfp4_mxfp8_quantize_elem(m8, 4, 64, e, p, p, st), MIS);
    EXPECT(nvfp4_mxfp8_quantize_elem(p, 4, 64, e, m8, p, st), MIS);
    EXPECT(nvfp4_mxfp8_quantize_elem(p, 0, 64, e, p, p, st), OK);
    EXPECT(nvfp4_mxfp8_gemm_elem(nullptr, p, e, p, p, e, 4, 4, 128, p, st), VAL);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, p, e, p, p, e, 4, 4, 64, p, st), SHAPE);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, p, e, p, p, e, 4, -1, 128, p, st), SHAPE);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, p, e, m8, p, e, 4, 4, 128, p, st), MIS);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, m2, e, p, p, e, 4, 4, 128, p, st), MIS);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, p, e, p, p, e, 0, 4, 128, p, st), OK);
  }
  for (int bad : {-1, 2, 7, 1 << 30}) {
    EXPECT(nvfp4_mxfp8_quantize_elem(p, 4, 64, bad, p, p, st), VAL);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, p, bad, p, p, 0, 4, 4, 128, p, st), VAL);
    EXPECT(nvfp4_mxfp8_gemm_elem(p, p, 0, p, p, bad, 4, 4, 128, p, st), VAL);
  }
  EXPECT(nvfp4_mxfp8_quantize(nullptr, 4, 64, p, p, st), VAL);
  EXPECT(nvfp4_mxfp8_gemm(p, p, p, p, 4, 4, 64, p, st), SHAPE);

  // ---- rowwise FP8 ----
  EXPECT(nvfp4_fp8r_quantize(nullptr, 4, 64, p, p, st), VAL);
  EXPECT(nvfp4_fp8r_quantize(p, 4, 64, p, nullptr, st), VAL);
  EXPECT(nvfp4_fp8r_quantize(p, -4, 64, p, p, st), SHAPE);
  EXPECT(nvfp4_fp8r_quantize(m8, 4, 64, p, p, st), MIS);
  EXPECT(nvfp4_fp8r_quantize(p, 0, 64, p, p, st), OK);
  EXPECT(nvfp4_fp8r_gemm(p, p, p, nullptr, 4, 4, 128, p, st), VAL);
  EXPECT(nvfp4_fp8r_gemm(p, p, p, p, 4, 4, 64, p, st), SHAPE);
  EXPECT(nvfp4_fp8r_gemm(p, p, m8, p, 4, 4, 128, p, st), MIS);
  EXPECT(nvfp4_fp8r_gemm(p, p, p, p, 4, 0, 128, p, st), OK);

  // ---- linear, its plan and workspace, the allocation-free form ----
  const size_t wsb = nvfp4_linear_workspace_bytes(4, 64);
  EXPECT_TRUE(wsb > 0 && wsb <= sizeof(g_buf));
  EXPECT_TRUE(nvfp4_linear_workspace_bytes(-1, 64) == 0);
  EXPECT_TRUE(nvfp4_linear_workspace_bytes(4, 40) == 0);
  EXPECT_TRUE(nvfp4_linear_workspace_bytes(INT64_MAX, 16) == 0);
  EXPECT(nvfp4_linear(nullptr, gs, p, p, gs, 4, 4, 64, p, p, wsb, st), VAL);
  EXPECT(nvfp4_linear(p, gs, nullptr, p, gs, 4, 4, 64, p, p, wsb, st), VAL);
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 4, 4, 64, nullptr, p, wsb, st), VAL);
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 4, 4, 64, p, nullptr, wsb, st), VAL);
  for (float b : kBadScales) {
    EXPECT(nvfp4_linear(p, b, p, p, gs, 4, 4, 64, p, p, wsb, st), VAL);
    EXPECT(nvfp4_linear(p, gs, p, p, b, 4, 4, 64, p, p, wsb, st), VAL);
  }
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 4, 4, 64, p, p, wsb - 1, st), WS);
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 4, 4, 64, p, p, 0, st), WS);
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 4, 4, 64, p, m8, wsb, st), MIS);
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 4, 4, 40, p, p, wsb, st), SHAPE);
  EXPECT(nvfp4_linear(p, gs, p, p, gs, 0, 4, 64, p, p, 0, st), OK);
  EXPECT(nvfp4_linear_plan(4, 4, 64, 0, nullptr), VAL);
  EXPECT(nvfp4_linear_noalloc(nullptr, gs, p, p, gs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_linear_noalloc(p, gs, p, p, gs, 4855, 64, 12288, p, st), BIG);
  EXPECT(nvfp4_linear_noalloc(p, gs, p, p, gs, (int64_t)1 << 30, 64, 1024, p, st), BIG);
  EXPECT(nvfp4_linear_noalloc(p, gs, p, p, gs, 4, 4, 40, p, st), SHAPE);
  for (float b : kBadScales) EXPECT(nvfp4_linear_noalloc(p, b, p, p, gs, 4, 4, 64, p, st), VAL);

  // ---- calibration and device-resident scales ----
  EXPECT(nvfp4_amax(nullptr, 64, dgs, st), VAL);
  EXPECT(nvfp4_amax(p, 64, nullptr, st), VAL);
  EXPECT(nvfp4_amax(p, -1, dgs, st), SHAPE);
  EXPECT(nvfp4_amax(m8, 64, dgs, st), MIS);
  EXPECT(nvfp4_amax(p, 64, (float*)(g_buf + 2), st), MIS);
  EXPECT(nvfp4_calibrate_device(nullptr, 64, dgs, st), VAL);
  EXPECT(nvfp4_calibrate_device(p, 64, nullptr, st), VAL);
  EXPECT(nvfp4_calibrate_device(p, -1, dgs, st), SHAPE);
  EXPECT(nvfp4_quantize_devgs(p, 4, 64, nullptr, p, p, st), VAL);
  EXPECT(nvfp4_quantize_devgs(p, 4, 40, dgs, p, p, st), SHAPE);
  EXPECT(nvfp4_quantize_devgs(p, 4, 64, (const float*)(g_buf + 2), p, p, st), MIS);
  EXPECT(nvfp4_gemm_devgs(p, p, nullptr, p, p, dgs, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm_devgs(p, p, dgs, p, p, nullptr, 4, 4, 64, p, st), VAL);
  EXPECT(nvfp4_gemm_devgs(p, p, dgs, p, p, dgs, 4, 4, 40, p, st), SHAPE);
  EXPECT(nvfp4_linear_devgs(p, nullptr, p, p, dgs, 4, 4, 64, p, p, wsb, st), VAL);
  EXPECT(nvfp4_linear_devgs(p, dgs, p, p, dgs, 4, 4, 64, p, p, wsb - 1, st), WS);

  // ---- shape fuzz over extreme values: plans and sizes must not overflow, and each
  // entry point must reject exactly the shapes its plan rejects ----
  const std::vector<int64_t> vals = {INT64_MIN, -((int64_t)1 << 40), -17, -1, 0, 1, 15, 16, 17, 31,
                                     32, 48, 64, 96, 128, 4608, ((int64_t)1 << 22) + 32,
                                     ((int64_t)1 << 31) - 1, (int64_t)1 << 31,
                                     ((int64_t)1 << 32) + 16, (int64_t)1 << 40, (int64_t)1 << 61,
                                     ((int64_t)1 << 62) + 16, INT64_MAX - 15, INT64_MAX};
  for (int64_t M : vals)
    for (int64_t N : vals)
      for (int64_t K : vals) {
        for (int cus : {0, 1, 32, 256, 1 << 20}) {
          int k1 = -1, k2 = -1, f = -1;
          const int s1 = nvfp4_gemm_plan(M, N, K, cus, &k1);
          const int s2 = nvfp4_gemm_w4a16_plan(M, N, K, cus, &k2);
          const int s3 = nvfp4_linear_plan(M, N, K, cus, &f);
          EXPECT_TRUE(s1 == OK || s1 == SHAPE);
          EXPECT_TRUE(s2 == OK || s2 == SHAPE);
          EXPECT_TRUE(s3 == OK || s3 == SHAPE);
          if (s1 == OK) EXPECT_TRUE(k1 >= 0 && k1 <= 9);
          if (s2 == OK) EXPECT_TRUE(k2 >= 0 && k2 <= 8);
          if (s3 == OK) EXPECT_TRUE(f == 0 || f == 1);
          if (cus != 0) continue;
          // rejected shapes fail the same way in the entry points (accepted ones would reach
          // the device, so only the rejections are called)
          if (s1 == SHAPE) EXPECT(nvfp4_gemm(p, p, gs, p, p, gs, M, N, K, p, st), SHAPE);
          if (s2 == SHAPE) EXPECT(nvfp4_gemm_w4a16(p, p, p, gs, M, N, K, p, st), SHAPE);
          if (s3 == SHAPE) EXPECT(nvfp4_linear(p, gs, p, p, gs, M, N, K, p, p, sizeof(g_buf), st), SHAPE);
        }
        const size_t b = nvfp4_linear_workspace_bytes(M, K);
        int f = -1;
        if (b == 0) EXPECT_TRUE(nvfp4_linear_plan(M, 16, K, 0, &f) == SHAPE || M == 0);
      }

  printf("checks %ld failures %ld\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
