// C ABI of libnvfp4: argument validation, device check and kernel dispatch.
// The entry points and their contracts are declared in include/nvfp4.h and
// include/nvfp4_selftest.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/nvfp4.h"
#include "../../include/nvfp4_selftest.h"
#include "kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;

struct DeviceEntry {
  std::once_flag once;
  int status = NVFP4_ERROR_UNSUPPORTED_DEVICE;
  hipError_t err = hipSuccess;
  nvfp4::LaunchInfo info{0, 0};
};
DeviceEntry g_devices[kMaxDevices];

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return NVFP4_ERROR_HIP;
}

// Current device must be gfx950; the answer is cached per device (thread-safe).
int current_device(nvfp4::LaunchInfo* info) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip_error = (int)e;
    return NVFP4_ERROR_UNSUPPORTED_DEVICE;
  }
  if (dev >= kMaxDevices) return NVFP4_ERROR_UNSUPPORTED_DEVICE;
  DeviceEntry& d = g_devices[dev];
  std::call_once(d.once, [&]() {
    hipDeviceProp_t prop;
    d.err = hipGetDeviceProperties(&prop, dev);
    if (d.err != hipSuccess) {
      d.status = NVFP4_ERROR_HIP;
      return;
    }
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      d.status = NVFP4_ERROR_UNSUPPORTED_DEVICE;
      return;
    }
    d.info.num_cus = prop.multiProcessorCount;
    d.info.device = dev;
    d.status = NVFP4_SUCCESS;
  });
  if (d.status == NVFP4_ERROR_HIP) g_last_hip_error = (int)d.err;
  *info = d.info;
  return d.status;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Static device scratch of nvfp4_linear_noalloc: the workspace of nvfp4_linear (quantized
// activations), for callers that cannot allocate. Every device the library is loaded on
// holds its own copy until the process ends. In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchEntry {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
ScratchEntry g_scratch[kMaxDevices];

// Device address of this device's scratch (info.device is current).
int scratch_pointer(const nvfp4::LaunchInfo& info, void** out) {
  ScratchEntry& e = g_scratch[info.device];
  std::call_once(e.once, [&]() {
    void* p = nullptr;
    e.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    e.ptr = e.err == hipSuccess ? p : nullptr;
  });
  if (e.err != hipSuccess || e.ptr == nullptr) {
    g_last_hip_error = (int)(e.err != hipSuccess ? e.err : hipErrorInvalidSymbol);
    return NVFP4_ERROR_HIP;
  }
  *out = e.ptr;
  return NVFP4_SUCCESS;
}

// Global scales: finite, in [2^-90, 2^90]. In this range every per-block divisor
// d = s * gs (s >= 2^-9) and 6 * gs stay far enough from the fp32 subnormal range that
// the quantizer's reciprocal-plus-correction divisions are exact (their residuals never
// underflow).
bool valid_scale(float g) { return isfinite(g) && g >= 0x1p-90f && g <= 0x1p90f; }

// Shape: rows >= 0, K >= 16, K % 16 == 0, rows * K without overflow (bytes < 2^62).
int check_shape(int64_t rows, int64_t K) {
  if (rows < 0 || K < 16 || K % 16 != 0) return NVFP4_ERROR_INVALID_SHAPE;
  if (rows > 0 && K > ((int64_t)1 << 61) / rows) return NVFP4_ERROR_INVALID_SHAPE;
  return NVFP4_SUCCESS;
}

constexpr size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int validate_gemm(const void* ap, const void* as, float ags, const void* wp, const void* ws,
                  float wgs, int64_t M, int64_t N, int64_t K, const void* out) {
  if (!ap || !as || !wp || !ws || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (!valid_scale(ags) || !valid_scale(wgs)) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  s = check_shape(N, K);
  if (s) return s;
  if (M > 0 && N > ((int64_t)1 << 61) / M) return NVFP4_ERROR_INVALID_SHAPE;
  if (!aligned(ap, 16) || !aligned(wp, 16) || !aligned(out, 16) || !aligned(as, 4) ||
      !aligned(ws, 4))
    return NVFP4_ERROR_MISALIGNED;
  return NVFP4_SUCCESS;
}

// Shape rules of nvfp4_gemm_w4a16 (its status, 0 when accepted).
int check_w4a16_shape(int64_t M, int64_t N, int64_t K) {
  int s = check_shape(M, K);
  if (s) return s;
  s = check_shape(N, K);
  if (s) return s;
  if (K % 32 != 0 || K > ((int64_t)1 << 22)) return NVFP4_ERROR_INVALID_SHAPE;
  if (M > 0 && N > ((int64_t)1 << 61) / M) return NVFP4_ERROR_INVALID_SHAPE;
  return NVFP4_SUCCESS;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_SUCCESS: return "success";
    case NVFP4_ERROR_INVALID_VALUE: return "invalid value (null pointer or bad global scale)";
    case NVFP4_ERROR_INVALID_SHAPE: return "invalid shape (need K >= 16, K % 16 == 0, sizes >= 0)";
    case NVFP4_ERROR_MISALIGNED: return "misaligned pointer";
    case NVFP4_ERROR_WORKSPACE: return "workspace too small";
    case NVFP4_ERROR_UNSUPPORTED_DEVICE: return "no gfx950 device";
    case NVFP4_ERROR_HIP: return "HIP runtime error";
    case NVFP4_ERROR_TOO_LARGE:
      return "problem needs more than the static scratch of nvfp4_linear_noalloc (32 MiB)";
    default: return "unknown status";
  }
}

int nvfp4_last_hip_error(void) { return g_last_hip_error; }

float nvfp4_global_scale_from_amax(float amax) {
  if (!isfinite(amax) || amax < 0.0f) return NAN;
  if (amax == 0.0f) return 1.0f;
  volatile float den = 2688.0f;  // 6 * 448, exact
  return amax / den;             // IEEE binary32 division
}

int nvfp4_quantize(const void* x, int64_t M, int64_t K, float gs, void* packed, void* scales,
                   void* stream) {
  if (!x || !packed || !scales) return NVFP4_ERROR_INVALID_VALUE;
  if (!valid_scale(gs)) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return NVFP4_ERROR_MISALIGNED;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_quantize(x, M, K, gs, packed, scales, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_gemm(const void* ap, const void* as, float ags, const void* wp, const void* ws, float wgs,
               int64_t M, int64_t N, int64_t K, void* out, void* stream) {
  int s = validate_gemm(ap, as, ags, wp, ws, wgs, M, N, K, out);
  if (s) return s;
  if (M == 0 || N == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  const nvfp4::Alpha al = nvfp4::split_alpha(ags, wgs);
  nvfp4::GemmProblem p{(const uint8_t*)ap, (const uint8_t*)as, (const uint8_t*)wp,
                       (const uint8_t*)ws, (uint16_t*)out, M, N, K, al.m, nullptr, nullptr, al.e};
  hipError_t e = nvfp4::launch_gemm(p, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_gemm_plan(int64_t M, int64_t N, int64_t K, int num_cus, int* kernel) {
  if (!kernel) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  s = check_shape(N, K);
  if (s) return s;
  if (M > 0 && N > ((int64_t)1 << 61) / M) return NVFP4_ERROR_INVALID_SHAPE;
  *kernel = nvfp4::plan_gemm(M, N, K, true, num_cus).kernel;
  return NVFP4_SUCCESS;
}

int nvfp4_gemm_w4a16_plan(int64_t M, int64_t N, int64_t K, int num_cus, int* kernel) {
  if (!kernel) return NVFP4_ERROR_INVALID_VALUE;
  const int s = check_w4a16_shape(M, N, K);
  if (s) return s;
  *kernel = (int)nvfp4::plan_gemm_w4a16(M, N, K, num_cus, true);
  return NVFP4_SUCCESS;
}

int nvfp4_gemm_w4a16(const void* x, const void* wp, const void* ws, float wgs, int64_t M,
                     int64_t N, int64_t K, void* out, void* stream) {
  if (!x || !wp || !ws || !out) return NVFP4_ERROR_INVALID_VALUE;
  if (!valid_scale(wgs)) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_w4a16_shape(M, N, K);
  if (s) return s;
  if (!aligned(x, 16) || !aligned(wp, 16) || !aligned(out, 16) || !aligned(ws, 4))
    return NVFP4_ERROR_MISALIGNED;
  if (M == 0 || N == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  nvfp4::W4A16Problem p{(const uint16_t*)x, (const uint8_t*)wp, (const uint8_t*)ws,
                        (uint16_t*)out, M, N, K, wgs};
  hipError_t e = nvfp4::launch_gemm_w4a16(p, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_mxfp8_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                         void* stream) {
  return nvfp4_mxfp8_quantize_elem(x, M, K, NVFP4_MX_E4M3, codes, scales, stream);
}

int nvfp4_mxfp8_quantize_elem(const void* x, int64_t M, int64_t K, int element, void* codes,
                              void* scales, void* stream) {
  if (!x || !codes || !scales) return NVFP4_ERROR_INVALID_VALUE;
  if (element != NVFP4_MX_E4M3 && element != NVFP4_MX_E5M2) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  if (K % 32 != 0) return NVFP4_ERROR_INVALID_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 16)) return NVFP4_ERROR_MISALIGNED;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_mx_quantize(x, M, K, codes, scales, (hipStream_t)stream, info,
                                           (nvfp4::MxElement)element);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_mxfp8_gemm(const void* ac, const void* as, const void* wc, const void* ws, int64_t M,
                     int64_t N, int64_t K, void* out, void* stream) {
  return nvfp4_mxfp8_gemm_elem(ac, as, NVFP4_MX_E4M3, wc, ws, NVFP4_MX_E4M3, M, N, K, out, stream);
}

int nvfp4_mxfp8_gemm_elem(const void* ac, const void* as, int a_element, const void* wc,
                          const void* ws, int w_element, int64_t M, int64_t N, int64_t K,
                          void* out, void* stream) {
  if (!ac || !as || !wc || !ws || !out) return NVFP4_ERROR_INVALID_VALUE;
  if ((a_element != NVFP4_MX_E4M3 && a_element != NVFP4_MX_E5M2) ||
      (w_element != NVFP4_MX_E4M3 && w_element != NVFP4_MX_E5M2))
    return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  s = check_shape(N, K);
  if (s) return s;
  if (K % 128 != 0) return NVFP4_ERROR_INVALID_SHAPE;
  if (M > 0 && N > ((int64_t)1 << 61) / M) return NVFP4_ERROR_INVALID_SHAPE;
  // 32-bit buffer offsets, with one 256-row tile past the end
  if (!nvfp4::fits_i31(M + 256, K) || !nvfp4::fits_i31(N + 256, K))
    return NVFP4_ERROR_INVALID_SHAPE;
  if (!aligned(ac, 16) || !aligned(wc, 16) || !aligned(out, 16) || !aligned(as, 4) ||
      !aligned(ws, 4))
    return NVFP4_ERROR_MISALIGNED;
  if (M == 0 || N == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  nvfp4::GemmProblem p{(const uint8_t*)ac, (const uint8_t*)as, (const uint8_t*)wc,
                       (const uint8_t*)ws, (uint16_t*)out, M, N, K, 1.0f};
  hipError_t e = nvfp4::launch_mx_gemm(p, (hipStream_t)stream, info, (nvfp4::MxElement)a_element,
                                       (nvfp4::MxElement)w_element);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_fp8r_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                        void* stream) {
  if (!x || !codes || !scales) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return NVFP4_ERROR_MISALIGNED;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_fp8r_quantize(x, M, K, codes, scales, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_fp8r_gemm(const void* ac, const void* as, const void* wc, const void* ws, int64_t M,
                    int64_t N, int64_t K, void* out, void* stream) {
  if (!ac || !as || !wc || !ws || !out) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  s = check_shape(N, K);
  if (s) return s;
  if (K % 128 != 0) return NVFP4_ERROR_INVALID_SHAPE;
  if (M > 0 && N > ((int64_t)1 << 61) / M) return NVFP4_ERROR_INVALID_SHAPE;
  // 32-bit buffer offsets, with one 256-row tile past the end (codes and fp32 scales)
  if (!nvfp4::fits_i31(M + 256, K) || !nvfp4::fits_i31(N + 256, K))
    return NVFP4_ERROR_INVALID_SHAPE;
  if (!aligned(ac, 16) || !aligned(wc, 16) || !aligned(out, 16) || !aligned(as, 4) ||
      !aligned(ws, 4))
    return NVFP4_ERROR_MISALIGNED;
  if (M == 0 || N == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  nvfp4::GemmProblem p{(const uint8_t*)ac, (const uint8_t*)as, (const uint8_t*)wc,
                       (const uint8_t*)ws, (uint16_t*)out, M, N, K, 1.0f};
  hipError_t e = nvfp4::launch_fp8r_gemm(p, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K) {
  if (check_shape(M, K)) return 0;
  return round_up((size_t)(M * K / 2), 256) + round_up((size_t)(M * K / 16), 256);
}

}  // extern "C"

namespace {

// The launches of nvfp4_linear once its arguments are valid and M > 0: quantize into the
// workspace, then the GEMM (or the one fused kernel for the shortest activations).
int linear_launch(const void* x, float ags, const void* wp, const void* ws, float wgs, int64_t M,
                  int64_t N, int64_t K, void* out, void* workspace, void* stream,
                  const nvfp4::LaunchInfo& info) {
  const size_t packed_bytes = round_up((size_t)(M * K / 2), 256);
  uint8_t* ap = (uint8_t*)workspace;
  uint8_t* as = ap + packed_bytes;
  const nvfp4::Alpha al = nvfp4::split_alpha(ags, wgs);
  nvfp4::GemmProblem p{ap, as, (const uint8_t*)wp, (const uint8_t*)ws, (uint16_t*)out,
                       M, N, K, al.m, nullptr, nullptr, al.e};
  hipError_t e;
  if (N > 0 && nvfp4::linear_fused(M, N, K, true, info.num_cus)) {
    const float den = 6.0f * ags;
    const nvfp4::FusedQuant fq{x, ags, den, 1.0f / den, nullptr, ap, as};
    e = nvfp4::launch_linear_fused(p, fq, (hipStream_t)stream, info.num_cus);
    return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
  }
  e = nvfp4::launch_quantize(x, M, K, ags, ap, as, (hipStream_t)stream, info);
  if (e != hipSuccess) return hip_fail(e);
  if (N == 0) return NVFP4_SUCCESS;
  e = nvfp4::launch_gemm(p, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

// Argument checks shared by nvfp4_linear and nvfp4_linear_noalloc (the workspace address
// only enters through its alignment).
int validate_linear(const void* x, float ags, const void* wp, const void* ws, float wgs, int64_t M,
                    int64_t N, int64_t K, const void* out, const void* workspace) {
  if (!x || !workspace) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  const uint8_t* ap = (const uint8_t*)workspace;
  s = validate_gemm(ap, ap + round_up((size_t)(M * K / 2), 256), ags, wp, ws, wgs, M, N, K, out);
  if (s) return s;
  if (!aligned(x, 16)) return NVFP4_ERROR_MISALIGNED;
  return NVFP4_SUCCESS;
}

}  // namespace

extern "C" {

int nvfp4_linear(const void* x, float ags, const void* wp, const void* ws, float wgs, int64_t M,
                 int64_t N, int64_t K, void* out, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int s = validate_linear(x, ags, wp, ws, wgs, M, N, K, out, workspace);
  if (s) return s;
  if (workspace_bytes < nvfp4_linear_workspace_bytes(M, K)) return NVFP4_ERROR_WORKSPACE;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  return linear_launch(x, ags, wp, ws, wgs, M, N, K, out, workspace, stream, info);
}

int nvfp4_linear_noalloc(const void* x, float ags, const void* wp, const void* ws, float wgs,
                         int64_t M, int64_t N, int64_t K, void* out, void* stream) {
  // a stand-in workspace address for the checks (the scratch is 256-byte aligned)
  static const uint8_t kAligned[256] __attribute__((aligned(256))) = {0};
  int s = validate_linear(x, ags, wp, ws, wgs, M, N, K, out, kAligned);
  if (s) return s;
  if (nvfp4_linear_workspace_bytes(M, K) > kScratchBytes) return NVFP4_ERROR_TOO_LARGE;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  void* work = nullptr;
  s = scratch_pointer(info, &work);
  if (s) return s;
  return linear_launch(x, ags, wp, ws, wgs, M, N, K, out, work, stream, info);
}

int nvfp4_linear_plan(int64_t M, int64_t N, int64_t K, int num_cus, int* fused) {
  if (!fused) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  s = check_shape(N, K);
  if (s) return s;
  if (M > 0 && N > ((int64_t)1 << 61) / M) return NVFP4_ERROR_INVALID_SHAPE;
  *fused = (M > 0 && N > 0 && nvfp4::linear_fused(M, N, K, true, num_cus)) ? 1 : 0;
  return NVFP4_SUCCESS;
}

int nvfp4_amax(const void* x, int64_t n, float* amax_out, void* stream) {
  if (!x || !amax_out) return NVFP4_ERROR_INVALID_VALUE;
  if (n < 0) return NVFP4_ERROR_INVALID_SHAPE;
  if (!aligned(x, 16) || !aligned(amax_out, 4)) return NVFP4_ERROR_MISALIGNED;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_amax(x, n, amax_out, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

// ---- device-resident global scales -------------------------------------------------------

int nvfp4_calibrate_device(const void* x, int64_t n, float* gs_device, void* stream) {
  if (!x || !gs_device) return NVFP4_ERROR_INVALID_VALUE;
  if (n < 0) return NVFP4_ERROR_INVALID_SHAPE;
  if (!aligned(x, 16) || !aligned(gs_device, 4)) return NVFP4_ERROR_MISALIGNED;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_calibrate(x, n, gs_device, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_quantize_devgs(const void* x, int64_t M, int64_t K, const float* gs_device, void* packed,
                         void* scales, void* stream) {
  if (!x || !packed || !scales || !gs_device) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(gs_device, 4))
    return NVFP4_ERROR_MISALIGNED;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_quantize(x, M, K, 1.0f, packed, scales, (hipStream_t)stream, info,
                                        gs_device);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_gemm_devgs(const void* ap, const void* as, const float* ags_device, const void* wp,
                     const void* ws, const float* wgs_device, int64_t M, int64_t N, int64_t K,
                     void* out, void* stream) {
  if (!ags_device || !wgs_device) return NVFP4_ERROR_INVALID_VALUE;
  if (!aligned(ags_device, 4) || !aligned(wgs_device, 4)) return NVFP4_ERROR_MISALIGNED;
  int s = validate_gemm(ap, as, 1.0f, wp, ws, 1.0f, M, N, K, out);
  if (s) return s;
  if (M == 0 || N == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  nvfp4::GemmProblem p{(const uint8_t*)ap, (const uint8_t*)as, (const uint8_t*)wp,
                       (const uint8_t*)ws, (uint16_t*)out, M, N, K, 1.0f, ags_device, wgs_device};
  hipError_t e = nvfp4::launch_gemm(p, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_linear_devgs(const void* x, const float* ags_device, const void* wp, const void* ws,
                       const float* wgs_device, int64_t M, int64_t N, int64_t K, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !workspace || !ags_device || !wgs_device) return NVFP4_ERROR_INVALID_VALUE;
  int s = check_shape(M, K);
  if (s) return s;
  const size_t packed_bytes = round_up((size_t)(M * K / 2), 256);
  uint8_t* ap = (uint8_t*)workspace;
  uint8_t* as = ap + packed_bytes;
  s = validate_gemm(ap, as, 1.0f, wp, ws, 1.0f, M, N, K, out);
  if (s) return s;
  if (!aligned(x, 16) || !aligned(ags_device, 4) || !aligned(wgs_device, 4))
    return NVFP4_ERROR_MISALIGNED;
  if (workspace_bytes < nvfp4_linear_workspace_bytes(M, K)) return NVFP4_ERROR_WORKSPACE;
  if (M == 0) return NVFP4_SUCCESS;
  nvfp4::LaunchInfo info;
  s = current_device(&info);
  if (s) return s;
  nvfp4::GemmProblem p{ap, as, (const uint8_t*)wp, (const uint8_t*)ws, (uint16_t*)out,
                       M, N, K, 1.0f, ags_device, wgs_device};
  hipError_t e;
  if (N > 0 && nvfp4::linear_fused(M, N, K, true, info.num_cus)) {
    const nvfp4::FusedQuant fq{x, 1.0f, 6.0f, 1.0f / 6.0f, ags_device, ap, as};
    e = nvfp4::launch_linear_fused(p, fq, (hipStream_t)stream, info.num_cus);
    return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
  }
  e = nvfp4::launch_quantize(x, M, K, 1.0f, ap, as, (hipStream_t)stream, info, ags_device);
  if (e != hipSuccess) return hip_fail(e);
  if (N == 0) return NVFP4_SUCCESS;
  e = nvfp4::launch_gemm(p, (hipStream_t)stream, info);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

// ---- self-test entry points ----------------------------------------------------------

int nvfp4_selftest_e2m1_encode(const float* y, uint8_t* hw_codes, uint8_t* sw_codes, int64_t n,
                               void* stream) {
  if (!y || !hw_codes || !sw_codes) return NVFP4_ERROR_INVALID_VALUE;
  if (n < 0) return NVFP4_ERROR_INVALID_SHAPE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_selftest_encode(y, hw_codes, sw_codes, n, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_e2m1_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                   void* stream) {
  if (!mismatches || !first16) return NVFP4_ERROR_INVALID_VALUE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_selftest_encode_exhaustive(mismatches, first16, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_mxfp8_e4m3_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                         void* stream) {
  if (!mismatches || !first16) return NVFP4_ERROR_INVALID_VALUE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e =
      nvfp4::launch_mx_selftest_e4m3_exhaustive(mismatches, first16, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_mxfp8_e5m2_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                         void* stream) {
  if (!mismatches || !first16) return NVFP4_ERROR_INVALID_VALUE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e =
      nvfp4::launch_mx_selftest_e5m2_exhaustive(mismatches, first16, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_bf16_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                   void* stream) {
  if (!mismatches || !first16) return NVFP4_ERROR_INVALID_VALUE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_selftest_bf16_exhaustive(mismatches, first16, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_division(unsigned long long* mismatches, uint32_t* first16, void* stream) {
  if (!mismatches || !first16) return NVFP4_ERROR_INVALID_VALUE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_selftest_division(mismatches, first16, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_block_scale(const float* amax, float global_scale, uint8_t* codes, float* d,
                               int64_t n, void* stream) {
  if (!amax || !codes || !d) return NVFP4_ERROR_INVALID_VALUE;
  if (!valid_scale(global_scale)) return NVFP4_ERROR_INVALID_VALUE;
  if (n < 0) return NVFP4_ERROR_INVALID_SHAPE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_selftest_scale(amax, global_scale, codes, d, n, (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

int nvfp4_selftest_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* hw_f16,
                          uint16_t* sw_f16, int64_t nbytes, void* stream) {
  if (!packed || !scales || !hw_f16 || !sw_f16) return NVFP4_ERROR_INVALID_VALUE;
  if (nbytes < 0) return NVFP4_ERROR_INVALID_SHAPE;
  nvfp4::LaunchInfo info;
  int s = current_device(&info);
  if (s) return s;
  hipError_t e = nvfp4::launch_selftest_decode(packed, scales, hw_f16, sw_f16, nbytes,
                                               (hipStream_t)stream);
  return e == hipSuccess ? NVFP4_SUCCESS : hip_fail(e);
}

}  // extern "C"
