// Device helpers of the NVFP4 quantizer shared by the quantize kernel (quantize.hip) and
// the GEMM kernel that quantizes its own activations (gemm.hip): bf16 unpacking, the
// encode of 8 elements under a block scale, and the in-kernel global-scale setup.
#pragma once

#include "codec.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

__device__ __forceinline__ void unpack_bf16x8(const u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = u2f(w[i] << 16);
    f[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
  }
}

// Encode 8 values (in f) of one half block into 4 packed bytes (element 2j in the low
// nibble of byte j), given the block's scale. kClamp selects the quotient form that
// tolerates an overflowing |x| * r (only needed for blocks whose scale saturated).
template <bool kClamp>
__device__ __forceinline__ uint32_t encode_half(const float* f, const BlockScale& bs) {
  uint32_t out = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float y0 = kClamp ? div_by_scale(f[2 * j], bs.d, bs.r)
                            : div_by_scale_unclamped(f[2 * j], bs.d, bs.r);
    const float y1 = kClamp ? div_by_scale(f[2 * j + 1], bs.d, bs.r)
                            : div_by_scale_unclamped(f[2 * j + 1], bs.d, bs.r);
    switch (j) {
      case 0: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, y0, y1, 1.0f, 0); break;
      case 1: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, y0, y1, 1.0f, 1); break;
      case 2: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, y0, y1, 1.0f, 2); break;
      default: out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, y0, y1, 1.0f, 3); break;
    }
  }
  return out;
}

// Quotient constants of the global scale: den = RN(6 gs), rden = RN(1/den), computed on
// the host for a host scale; a global scale read from device memory is clamped
// (clamp_global_scale) and the constants are computed here with the same IEEE operations.
struct QuantScale {
  float gs, den, rden;
};
__device__ __forceinline__ QuantScale quant_scale(float gs, float den, float rden,
                                                  const float* gs_dev) {
  if (gs_dev != nullptr) {
    gs = clamp_global_scale(*gs_dev);
    den = 6.0f * gs;
    rden = 1.0f / den;
  }
  return QuantScale{gs, den, rden};
}

}  // namespace
}  // namespace nvfp4
