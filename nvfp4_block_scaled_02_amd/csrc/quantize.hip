// NVFP4 quantization kernel for gfx950: bf16 [M, K] -> packed E2M1 [M, K/2] + E4M3
// scales [M, K/16] under an fp32 global scale.
//
// The run-time activation quantizer that the pages pair with the FP4 GEMM
// ("BFL (fp8r / nvfp4)", Kernels table, nvfp4 row); microscaling with 16-element E2M1
// blocks (zubnet.ai page, paragraph 1).
//
// Design (memory-bound: 2 B read + 0.5625 B written per element):
//  * K % 16 == 0, so 16-element blocks never straddle rows and the tensor is a flat
//    array of M*K/16 independent blocks; block b reads bytes [32b, 32b+32) of x, writes
//    bytes [8b, 8b+8) of packed and byte b of scales.
//  * Two lanes share a block: lane 2i+h loads the h-th 16 bytes (8 elements) of block
//    i, so the lanes of a wave read 1 KiB of consecutive bytes per load instruction.
//    The block amax is the larger of the pair's partial maxima (one DPP lane swap);
//    both lanes derive the same scale, each encodes its 8 elements into one 32-bit word
//    (consecutive lanes write consecutive words) and the even lane writes the scale.
//  * Each lane handles UNROLL halves per step with all loads issued first, to keep
//    enough bytes in flight for HBM.
//  * Rounding: the per-block scale uses IEEE division; the per-element quotient
//    |x| / d uses the reciprocal of d plus Markstein's fma correction, which equals the
//    IEEE quotient for every bf16 x (see codec.hpp); the E2M1 encode is the gfx950
//    conversion instruction, whose rounding (to nearest even, saturating) is checked
//    exhaustively against the software encoder by the self-test entry points.
#include "quant_common.hpp"

namespace nvfp4 {

namespace {

// nhalves = 2 * (number of blocks); half index hi covers x[hi] (16 bytes) and packed
// word hi. The pair (hi, hi ^ 1) is one block; since nhalves is even and workgroups are
// a multiple of 2 lanes, both lanes of a pair are always in the same loop state.
template <int UNROLL>
__global__ void __launch_bounds__(256) quantize_kernel(const u32x4* __restrict__ x,
                                                       uint32_t* __restrict__ packed,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t nhalves, float gs, float den,
                                                       float rden, const float* gs_dev) {
  {
    const QuantScale qs = quant_scale(gs, den, rden, gs_dev);
    gs = qs.gs;
    den = qs.den;
    rden = qs.rden;
  }
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * UNROLL;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * UNROLL + threadIdx.x; base < nhalves;
       base += stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t hi = base + (int64_t)u * blockDim.x;
      v[u] = hi < nhalves ? __builtin_nontemporal_load(&x[hi]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t hi = base + (int64_t)u * blockDim.x;
      float f[8];
      unpack_bf16x8(v[u], f);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(f[i]));
      // partner lane's partial maximum (DPP quad_perm [1, 0, 3, 2]: lane ^ 1)
      const float o = __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false));
      const BlockScale bs = block_scale(__builtin_fmaxf(a, o), den, rden, gs);
      // Saturated scales are rare (the tensor's largest block under a self-calibrated
      // scale, or a static scale that is too small); the whole wave takes the clamped
      // quotient if any of its lanes has one.
      uint32_t word;
      if (__any(bs.code == kE4M3MaxCode))
        word = encode_half<true>(f, bs);
      else
        word = encode_half<false>(f, bs);
      if (hi < nhalves) {
        __builtin_nontemporal_store(word, &packed[hi]);
        if ((hi & 1) == 0) scales[hi >> 1] = (uint8_t)bs.code;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int64_t M, int64_t K, float gs, void* packed,
                           void* scales, hipStream_t stream, const LaunchInfo& dev,
                           const float* gs_dev) {
  const int64_t nhalves = M * (K / 16) * 2;
  if (nhalves == 0) return hipSuccess;
#ifndef NVFP4_QUANT_UNROLL
#define NVFP4_QUANT_UNROLL 2
#endif
#ifndef NVFP4_QUANT_WG_PER_CU
#define NVFP4_QUANT_WG_PER_CU 32
#endif
#ifndef NVFP4_QUANT_WG_PER_CU_SMALL
#define NVFP4_QUANT_WG_PER_CU_SMALL 6
#endif
  constexpr int kThreads = 256;
  constexpr int kUnroll = NVFP4_QUANT_UNROLL;
  const float den = 6.0f * gs;   // IEEE binary32 on the host
  const float rden = 1.0f / den;
  const int64_t want = (nhalves + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  // Enough workgroups to fill every CU several times over; the grid-stride loop covers
  // the rest.
  // Workgroups per compute unit: up to 2^21 half blocks (a 4608 x 3072 activation) fewer
  // workgroups that loop 2-3 times start sooner and finish together (8.64 -> 8.03 us there);
  // larger tensors stream best with many (4608 x 12288: 24.7 us at 32, 25.8-26.6 at 4-12).
  const int64_t per_cu = nhalves <= ((int64_t)1 << 21) ? NVFP4_QUANT_WG_PER_CU_SMALL : NVFP4_QUANT_WG_PER_CU;
  const int64_t cap = (int64_t)dev.num_cus * per_cu;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL((quantize_kernel<kUnroll>), dim3(grid), dim3(kThreads), 0, stream,
                     (const u32x4*)x, (uint32_t*)packed, (uint8_t*)scales, nhalves, gs, den, rden,
                     gs_dev);
  return hipGetLastError();
}

// ---- self-test support: the exact device functions the quantizer uses ---------------

namespace {

__global__ void selftest_encode_kernel(const float* __restrict__ y, uint8_t* __restrict__ hw,
                                       uint8_t* __restrict__ sw, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = y[i];
  hw[i] = (uint8_t)(__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu);
  sw[i] = (uint8_t)e2m1_encode_sw(v, v);
}

// All 2^32 binary32 patterns except NaNs: count where the conversion instruction and
// the software encoder disagree; record up to 16 offending patterns.
__global__ void selftest_encode_exhaustive_kernel(unsigned long long* __restrict__ count,
                                                  uint32_t* __restrict__ first) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t nthreads = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long local = 0;
  for (uint64_t u = tid; u < (1ull << 32); u += nthreads) {
    const uint32_t bits = (uint32_t)u;
    const float v = u2f(bits);
    if (v != v) continue;
    const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
    const uint32_t sw = e2m1_encode_sw(v, v);
    if (hw != sw) {
      const unsigned long long k = atomicAdd(count, 1ull);
      if (k < 16) first[k] = bits;
      ++local;
    }
  }
  (void)local;
}

// Markstein division vs IEEE division on every pair (bf16 significand of x, binary32
// significand of d), with x in [1, 4) and d in [1, 2).
__global__ void selftest_division_kernel(unsigned long long* __restrict__ count,
                                         uint32_t* __restrict__ first) {
  const uint32_t dm = blockIdx.x * blockDim.x + threadIdx.x;  // 2^23 threads
  if (dm >= (1u << 23)) return;
  const float d = u2f(0x3F800000u | dm);
  const float r = 1.0f / d;
  for (uint32_t xm = 0; xm < 260; ++xm) {
    // bf16 significands of x in [1, 4), then +0, -0 (whose quotient keeps the sign)
    const float x = xm < 256 ? u2f(((127u + (xm >> 7)) << 23) | ((xm & 127u) << 16))
                             : (xm & 1u ? -0.0f : 0.0f);
    const float y = xm < 258 ? div_by_scale(x, d, r) : div_by_scale(x, 0.0f, 0.0f);
    const float yu = xm < 258 ? div_by_scale_unclamped(x, d, r) : div_by_scale_unclamped(x, 0.0f, 0.0f);
    const float q = xm < 258 ? x / d : x;
    if (f2u(y) != f2u(q) || f2u(yu) != f2u(q)) {
      const unsigned long long k = atomicAdd(count, 1ull);
      if (k < 8) {
        first[2 * k] = f2u(x);
        first[2 * k + 1] = f2u(d);
      }
    }
  }
}

__global__ void selftest_scale_kernel(const float* __restrict__ amax, float gs, float den,
                                      float rden, uint8_t* __restrict__ code,
                                      float* __restrict__ d_out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const BlockScale b = block_scale(amax[i], den, rden, gs);
  code[i] = (uint8_t)b.code;
  d_out[i] = b.d;
}

}  // namespace

hipError_t launch_selftest_encode(const float* y, uint8_t* hw, uint8_t* sw, int64_t n,
                                  hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(selftest_encode_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, y, hw, sw, n);
  return hipGetLastError();
}

hipError_t launch_selftest_encode_exhaustive(unsigned long long* count, uint32_t* first,
                                             hipStream_t stream) {
  hipLaunchKernelGGL(selftest_encode_exhaustive_kernel, dim3(8192), dim3(256), 0, stream, count,
                     first);
  return hipGetLastError();
}

hipError_t launch_selftest_division(unsigned long long* count, uint32_t* first,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(selftest_division_kernel, dim3((1u << 23) / 256), dim3(256), 0, stream,
                     count, first);
  return hipGetLastError();
}

hipError_t launch_selftest_scale(const float* amax, float gs, uint8_t* code, float* d, int64_t n,
                                 hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const float den = 6.0f * gs;
  hipLaunchKernelGGL(selftest_scale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, amax, gs, den, 1.0f / den, code, d, n);
  return hipGetLastError();
}

}  // namespace nvfp4
