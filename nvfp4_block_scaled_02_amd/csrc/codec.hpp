// Scalar NVFP4 codecs shared by the quantize kernel, the GEMM decode and the self-test
// kernels. Everything here is plain IEEE binary32 / integer arithmetic; the functions
// marked NVFP4_HD compile for the host as well, so their rounding can be checked on a
// CPU. Hardware conversion builtins are device-only.
//
// Format: E2M1 elements, one E4M3 scale per 16-element block, fp32 global scale
// ("BFL (fp8r / nvfp4)", nvfp4 item; zubnet.ai page, paragraph 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define NVFP4_HD __host__ __device__ __forceinline__

namespace nvfp4 {

// Native 16- and 8-byte vectors (usable with the nontemporal load/store builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

NVFP4_HD float u2f(uint32_t u) {
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}
NVFP4_HD uint32_t f2u(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  return u;
}

// Largest E4M3 value and its code; largest E2M1 magnitude.
constexpr float kE4M3Max = 448.0f;
constexpr uint32_t kE4M3MaxCode = 0x7E;

// E4M3 code of the E4M3 value nearest to s (s >= 0, not NaN; +inf allowed), ties to
// the even code, saturating at 448 (0x7E).
//  * s >= 448: saturate.
//  * s < 2^-6 (E4M3 subnormal range, spacing 2^-9): code = round-half-even(s * 2^9);
//    the product is exact and code 8 is the smallest normal, so the rounding carries
//    into the normal range seamlessly.
//  * otherwise round the binary32 significand to 3 bits (half to even, at bit 20) and
//    rebias the exponent from 127 to 7.
NVFP4_HD uint32_t e4m3_encode_sat(float s) {
  if (!(s < kE4M3Max)) return kE4M3MaxCode;
  if (s < 0x1p-6f) return (uint32_t)__builtin_rintf(s * 512.0f);
  uint32_t b = f2u(s);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  return (b >> 20) - (120u << 3);
}

// Largest finite E5M2 value (1.75 * 2^15) and its code.
constexpr float kE5M2Max = 57344.0f;
constexpr uint32_t kE5M2MaxCode = 0x7B;

// E5M2 code of the E5M2 value nearest to s (s >= 0, not NaN; +inf allowed), ties to
// the even code, saturating at 57344 (0x7B).
//  * s >= 57344: saturate.
//  * s < 2^-14 (E5M2 subnormal range, spacing 2^-16): code = round-half-even(s * 2^16);
//    the product is exact and code 4 is the smallest normal, so the rounding carries
//    into the normal range seamlessly.
//  * otherwise round the binary32 significand to 2 bits (half to even, at bit 21) and
//    rebias the exponent from 127 to 15.
NVFP4_HD uint32_t e5m2_encode_sat(float s) {
  if (!(s < kE5M2Max)) return kE5M2MaxCode;
  if (s < 0x1p-14f) return (uint32_t)__builtin_rintf(s * 65536.0f);
  uint32_t b = f2u(s);
  b += 0xFFFFFu + ((b >> 21) & 1u);
  return (b >> 21) - (112u << 2);
}

// Exact value of a finite non-negative E4M3 code (0..0x7E), without relying on
// denormal arithmetic: subnormal codes are m * 2^-9, normal codes shift into a
// binary32 pattern with the exponent rebiased by +120.
NVFP4_HD float e4m3_decode(uint32_t c) {
  return c < 8u ? (float)c * 0x1p-9f : u2f((c << 20) + (120u << 23));
}

// E2M1 magnitude code of y >= 0 (or -0; +inf allowed): nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6. The midpoints
// 0.25, 1.25, 2.5, 5 go down (to codes 0, 2, 4, 6) and 0.75, 1.75, 3.5 go up (to codes
// 2, 4, 6).
NVFP4_HD uint32_t e2m1_magnitude_encode(float y) {
  return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
         (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
         (uint32_t)(y > 5.0f);
}

// Correctly rounded x / d for a bf16-valued x (8 significant bits) and a normal
// binary32 d, given r = RN(1/d) (Markstein's correction):
//   y0 = RN(x r),  e = RN(y0 d - x) (exact, fma),  y = RN(y0 - e r).
// An exhaustive check over every pair of significands (bf16 x, binary32 d) shows
// y == RN(x/d), and it stays exact while the residual e cannot underflow, which holds
// for every d = s * gs with s >= 2^-9 and gs >= 2^-90 in the quotient range that decides
// a code. Writing the residual as y0 d - x (not x - y0 d) keeps the sign of a zero x:
// for x = -0, e = +0 and y = -0 - (+0)r = -0. With r == 0 (for d == 0) the result is a
// zero carrying the sign of x.
//
// This form needs |x r| finite; it is used for every block whose scale did not saturate
// (there |x| / d <= amax / d < 9).
NVFP4_HD float div_by_scale_unclamped(float x, float d, float r) {
  const float y0 = x * r;
  const float e = __builtin_fmaf(y0, d, -x);
  return __builtin_fmaf(-e, r, y0);
}

NVFP4_HD float clamp8(float v) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_fmed3f(v, -8.0f, 8.0f);
#else
  return v < -8.0f ? -8.0f : (v > 8.0f ? 8.0f : v);
#endif
}

// Same quotient for any finite x: y0 is clamped to [-8, 8] first. Any |x/d| >= 6
// saturates the E2M1 code, so the clamp only keeps a huge quotient from turning into
// inf - inf = NaN; below 8 it changes nothing.
NVFP4_HD float div_by_scale(float x, float d, float r) {
  const float y0 = clamp8(x * r);
  const float e = __builtin_fmaf(y0, d, -x);
  return __builtin_fmaf(-e, r, y0);
}

// Per-block quantization state: the scale code, d = RN(s * gs) and r = RN(1/d) (0 when
// d == 0).
struct BlockScale {
  uint32_t code;
  float d;
  float r;
};

// Scale of one block from its amax under global scale gs, with den = RN(6 * gs) and
// rden = RN(1 / den): s_raw = RN(amax / den) (the same reciprocal-plus-correction
// quotient, amax being a bf16 value; the first product is clamped to [0, 1024] so an
// overflow ends in saturation, never NaN), code = E4M3(s_raw), d = RN(decode(code) * gs).
NVFP4_HD BlockScale block_scale(float amax, float den, float rden, float gs) {
  BlockScale b;
  float q0 = amax * rden;
  q0 = q0 < 1024.0f ? q0 : 1024.0f;
  const float e = __builtin_fmaf(q0, den, -amax);
  const float s_raw = __builtin_fmaf(-e, rden, q0);
  b.code = e4m3_encode_sat(s_raw);
  b.d = e4m3_decode(b.code) * gs;
  b.r = b.d == 0.0f ? 0.0f : 1.0f / b.d;
  return b;
}

// 4-bit code of one element (software path): sign bit of x, magnitude of |y|.
NVFP4_HD uint32_t e2m1_encode_sw(float x, float y) {
  uint32_t sign = (f2u(x) >> 31) << 3;
  return sign | e2m1_magnitude_encode(__builtin_fabsf(y));
}

// Global scales read from device memory: clamped into [2^-90, 2^90], the range in which
// the quantizer's divisions are exact (NaN, and anything not above 0, read as 1).
constexpr float kGsMin = 0x1p-90f, kGsMax = 0x1p90f;
NVFP4_HD float clamp_global_scale(float gs) {
  if (!(gs > 0.0f)) return 1.0f;
  return gs < kGsMin ? kGsMin : (gs > kGsMax ? kGsMax : gs);
}

}  // namespace nvfp4
