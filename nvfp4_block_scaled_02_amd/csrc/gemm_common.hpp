// Device helpers shared by the GEMM kernels (gemm.hip, gemm_w4a16.hip): operand decode
// of NVFP4 fragments, bf16 rounding of results and buffer resources.
#pragma once

#include "codec.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// f16 values {s(c0), s(c1)} of the two E4M3 scale codes in the low 16 bits of v (c0 in
// bits 0..7). Every E4M3 value, subnormals included, is a normal f16, so the
// conversion is exact.
template <bool kHw>
__device__ __forceinline__ half2_t scales_to_f16(uint32_t v) {
  if constexpr (kHw) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
  } else {
    half2_t r;
    r.x = (_Float16)e4m3_decode(v & 0xFFu);
    r.y = (_Float16)e4m3_decode((v >> 8) & 0xFFu);
    return r;
  }
}

// f16 high bytes of the E2M1 magnitudes 0, .5, 1, 1.5 | 2, 3, 4, 6 (low bytes are 0).
constexpr uint32_t kLutLo = 0x3E3C3800u;
constexpr uint32_t kLutHi = 0x46444240u;

// Eight E2M1 codes (element i in bits 4i..4i+3 of p) times the block scale s (both
// halves of s2), as f16. q and s are normal f16 values and q * s (at most 6
// significant bits, in [2^-10, 2688]) is a normal f16, so the product is exact.
template <bool kHw>
__device__ __forceinline__ half8_t decode8(uint32_t p, half2_t s2) {
  half2_t h[4];
  if constexpr (kHw) {
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 0);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 1);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 2);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(p, 1.0f, 3);
  } else {
    // Byte-table lookup: even elements from the low nibbles, odd from the high ones,
    // signs moved to bit 7 of each byte; then interleave into f16 high bytes.
    const uint32_t lo = __builtin_amdgcn_perm(kLutHi, kLutLo, p & 0x07070707u) |
                        ((p << 4) & 0x80808080u);
    const uint32_t hi = __builtin_amdgcn_perm(kLutHi, kLutLo, (p >> 4) & 0x07070707u) |
                        (p & 0x80808080u);
    h[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(hi, lo, 0x040C000Cu));
    h[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(hi, lo, 0x050C010Cu));
    h[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(hi, lo, 0x060C020Cu));
    h[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(hi, lo, 0x070C030Cu));
  }
  half8_t r;
  r.s01 = h[0] * s2;
  r.s23 = h[1] * s2;
  r.s45 = h[2] * s2;
  r.s67 = h[3] * s2;
  return r;
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t b = f2u(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Raw buffer resource over n bytes at p (gfx9-family descriptor word 3: 32-bit data
// format, no swizzle); loads at offsets >= n return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

}  // namespace
}  // namespace nvfp4
