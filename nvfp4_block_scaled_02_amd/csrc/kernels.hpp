// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

struct LaunchInfo {
  int num_cus;  // compute units of the current device
  int device;   // its index
};

// rows * row_bytes < 2^31 (a tile's 32-bit buffer offsets), for rows, row_bytes >= 0,
// evaluated without forming the product (which can exceed int64 for shapes the size
// checks accept, such as one row of 2^61 elements).
inline bool fits_i31(int64_t rows, int64_t row_bytes) {
  return row_bytes <= 0 || rows <= ((((int64_t)1) << 31) - 1) / row_bytes;
}

// gs_dev non-null: the global scale is read on the device from *gs_dev (clamped into
// [2^-90, 2^90], NaN read as 1) and `gs` is ignored.
hipError_t launch_quantize(const void* x, int64_t M, int64_t K, float gs, void* packed,
                           void* scales, hipStream_t stream, const LaunchInfo& dev,
                           const float* gs_dev = nullptr);

// The epilogue scale a_global * w_global as m * 2^e. When RN(a_global * w_global) is a
// normal binary32 (every realistic pair) m is that product and e = 0. Global scales in
// [2^-90, 2^90] can also multiply to anything in [2^-180, 2^180], where a single fp32
// alpha would be subnormal (precision lost) or infinite; then m is the rounded product of
// the two frexp mantissas, in [0.25, 1), e the sum of their exponents, and the epilogue
// applies 2^e with ldexp after the multiply by m.
struct Alpha {
  float m;
  int e;
};
__host__ __device__ inline Alpha split_alpha(float a, float w) {
  const float prod = a * w;
  if (prod >= 0x1p-126f && prod <= 0x1.fffffep127f) return Alpha{prod, 0};
  int ea = 0, ew = 0;
  const float ma = frexpf(a, &ea);
  const float mw = frexpf(w, &ew);
  return Alpha{ma * mw, ea + ew};
}

struct GemmProblem {
  const uint8_t* a_packed;
  const uint8_t* a_scales;
  const uint8_t* w_packed;
  const uint8_t* w_scales;
  uint16_t* out;
  int64_t M, N, K;
  float alpha;  // split_alpha(a_global, w_global): alpha * 2^alpha_exp
  // Device-resident global scales (both set, or both null): the kernel then reads both,
  // clamps each as the quantizer clamps a device-resident scale, and splits their product
  // with split_alpha; alpha and alpha_exp are unused.
  const float* a_gs_dev;
  const float* w_gs_dev;
  int alpha_exp = 0;
};

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev);

// The fused linear for short activations: the split-K GEMM quantizes its own bf16
// activations (bit-identical to launch_quantize) and, when ws_packed is set, the
// workgroups of the first weight-row tile store the codes and scales there. The GEMM
// problem's a_packed / a_scales are unused.
struct FusedQuant {
  const void* x;          // bf16 activations [M, K]
  float gs, den, rden;    // host global scale, RN(6 gs), RN(1 / RN(6 gs))
  const float* gs_dev;    // device-resident global scale instead (then gs/den/rden unused)
  uint8_t* ws_packed;     // [M, K/2] codes out, or null
  uint8_t* ws_scales;     // [M, K/16] scales out
};
bool linear_fused(int64_t M, int64_t N, int64_t K, bool aligned, int64_t cus);
hipError_t launch_linear_fused(const GemmProblem& p, const FusedQuant& fq, hipStream_t stream,
                               int64_t cus);

// The kernel launch_gemm picks for a shape (values of nvfp4_gemm_kernel in nvfp4.h), and
// the split-K workgroup shape (32a weight rows x 32b activation rows) when it splits.
struct SplitShape { int a, b; };
struct GemmPlan {
  int kernel;
  SplitShape split;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool aligned, int64_t cus,
                   bool allow_gemv16 = true);

// Weight rows per workgroup of the 16-row kernels (NVFP4 and W4A16): a multiple of 4 up
// to 16, the fewest that keep the grid within one workgroup per compute unit.
inline int gemv16_rows(int64_t N, int64_t cus) {
  const int64_t r = 4 * ((N + 4 * cus - 1) / (4 * cus));
  return (int)(r < 4 ? 4 : r > 16 ? 16 : r);
}

struct W4A16Problem {
  const uint16_t* x;  // bf16 [M, K]
  const uint8_t* w_packed;
  const uint8_t* w_scales;
  uint16_t* out;
  int64_t M, N, K;
  float alpha;  // the weights' global scale
};

// W4A16 kernels, in the order of the plan codes: split-K (short activations), the 288 x 192
// tile, the 256 x 256 tile, the tiles with their waves along N: 224 x 256, 128 x 256,
// 96 x 256, 128 x 128 and 64 x 128, and the 16-row kernel (at most 16 activation rows).
enum class W4A16Kernel {
  kSplitK = 0, kFit = 1, kTile256 = 2, kWide = 3, kWide128x256 = 4, kWide96x256 = 5,
  kWide128x128 = 6, kWide64x128 = 7, kGemv16 = 8
};
W4A16Kernel plan_gemm_w4a16(int64_t M, int64_t N, int64_t K, int64_t num_cus, bool aligned);
hipError_t launch_gemm_w4a16(const W4A16Problem& p, hipStream_t stream, const LaunchInfo& dev);

// MXFP8: codes/scales use GemmProblem's a_packed/a_scales/w_packed/w_scales (one byte
// per element, one E8M0 byte per 32 elements); alpha is 1. Elements are E4M3 or E5M2,
// each operand its own.
enum class MxElement { kE4M3 = 0, kE5M2 = 1 };
hipError_t launch_mx_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                              hipStream_t stream, const LaunchInfo& dev, MxElement elem);
hipError_t launch_mx_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev,
                          MxElement a_elem, MxElement w_elem);
// Rowwise FP8: codes as above, scales fp32 [rows] (GemmProblem's a_scales/w_scales point
// to fp32 arrays); alpha unused.
hipError_t launch_fp8r_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                                hipStream_t stream, const LaunchInfo& dev);
hipError_t launch_fp8r_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev);
hipError_t launch_mx_selftest_e4m3_exhaustive(unsigned long long* count, uint32_t* first,
                                              hipStream_t stream);
hipError_t launch_mx_selftest_e5m2_exhaustive(unsigned long long* count, uint32_t* first,
                                              hipStream_t stream);

hipError_t launch_amax(const void* x, int64_t n, float* out, hipStream_t stream,
                       const LaunchInfo& dev);
// amax of x, then in place the global scale from it: RN(amax / 2688) clamped into
// [2^-90, 2^90], 1 for amax == 0.
hipError_t launch_calibrate(const void* x, int64_t n, float* gs, hipStream_t stream,
                            const LaunchInfo& dev);

// self-test support
hipError_t launch_selftest_encode(const float* y, uint8_t* hw, uint8_t* sw, int64_t n,
                                  hipStream_t stream);
hipError_t launch_selftest_encode_exhaustive(unsigned long long* count, uint32_t* first,
                                             hipStream_t stream);
hipError_t launch_selftest_division(unsigned long long* count, uint32_t* first,
                                    hipStream_t stream);
hipError_t launch_selftest_scale(const float* amax, float gs, uint8_t* code, float* d, int64_t n,
                                 hipStream_t stream);
hipError_t launch_selftest_bf16_exhaustive(unsigned long long* count, uint32_t* first,
                                           hipStream_t stream);
hipError_t launch_selftest_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* hw,
                                  uint16_t* sw, int64_t nbytes, hipStream_t stream);

}  // namespace nvfp4
