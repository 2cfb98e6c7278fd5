// Rowwise FP8 ("fp8r") quantize for gfx950: bf16 [M, K] -> E4M3 codes [M, K] plus one
// fp32 scale per row.
//
// The scheme of the "BFL (fp8r / nvfp4)" page (scheme list, fp8r item): E4M3 weights with
// one fp32 scale per row, and activations quantized to E4M3 per row at run time. This
// library's reading: s = RN(amax / 448) (an all-zero row takes s = 1) and each element is
// the E4M3 value nearest to RN(x / s) (ties to even, clamped to +-448, sign copied).
//
// Memory-bound: 2 B read, 1 B written per element, plus 4 B per row; 16 bytes per lane
// and load (a wave's load instruction reads 1 KiB of consecutive bytes). Rows stay in
// registers: every load of the row is issued at once, the amax is reduced, and the codes
// are encoded from the registers (8 bytes per lane and group).
//  * K <= 2048: one wave per row (up to 4 loads per lane).
//  * 2048 < K <= 16384: one 256-thread workgroup per row (up to 8 loads per thread), the
//    four waves' maxima meeting in LDS. Splitting a long row over a workgroup keeps the
//    register count low, so enough workgroups are resident for one's encode to overlap
//    the others' loads and stores.
//  * Longer rows: one wave per row in two passes, the second reading the row again
//    (from L2).
//
// Rounding: the row scale is an IEEE division. The element quotient uses the reciprocal
// of s plus Markstein's fma correction (codec.hpp), which equals IEEE x / s for bf16 x and
// normal s while the residual cannot underflow; for every quotient that can decide a code
// (|x / s| >= 2^-11) that holds when s >= 2^-60, so rows with a smaller scale take the
// IEEE division instead. The E4M3 encode is gfx950's fp8 conversion, checked exhaustively
// against the software encoder by the MXFP8 self-test.
#include "codec.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

__device__ __forceinline__ float wave_max(float a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off, 64));
  return a;
}

// 8 elements of a row (one bf16x8 word) to 8 E4M3 codes under the row's scale.
__device__ __forceinline__ u32x2 encode8(const u32x4 v, float s, float r, bool corrected) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = u2f(w[i] << 16), x1 = u2f(w[i] & 0xFFFF0000u);
    y[2 * i] = corrected ? div_by_scale_unclamped(x0, s, r) : x0 / s;
    y[2 * i + 1] = corrected ? div_by_scale_unclamped(x1, s, r) : x1 / s;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_fmed3f(y[i], -kE4M3Max, kE4M3Max);
  uint32_t c0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  c0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c0, true);
  uint32_t c1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  c1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], c1, true);
  return u32x2{c0, c1};
}

__device__ __forceinline__ float amax8(const u32x4 v, float a) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a = __builtin_fmaxf(a, __builtin_fabsf(u2f(w[i] << 16)));
    a = __builtin_fmaxf(a, __builtin_fabsf(u2f(w[i] & 0xFFFF0000u)));
  }
  return a;
}

// Row scale s = RN(amax / 448) (1 for an all-zero row), stored by lane 0.
struct RowScale {
  float s, r;
  bool corrected;
};
__device__ __forceinline__ RowScale row_scale(float amax, float* scales, int64_t row, int lane) {
  RowScale rs;
  rs.s = amax > 0.0f ? amax / kE4M3Max : 1.0f;  // IEEE division
  if (lane == 0) scales[row] = rs.s;
  rs.r = 1.0f / rs.s;
  rs.corrected = rs.s >= 0x1p-60f;  // wave-uniform
  return rs;
}

// Rows of at most 64 * 8 * NR elements, held in registers.
template <int NR>
__global__ void __launch_bounds__(256) fp8r_quantize_regs_kernel(const u32x4* __restrict__ x,
                                                                 int64_t M, int64_t K,
                                                                 u32x2* __restrict__ codes,
                                                                 float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves
  const int ng = (int)(K >> 3);  // 8-element groups of the row
  const u32x4* xr = x + row * ng;
  u32x2* cr = codes + row * ng;
  u32x4 v[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int g = lane + 64 * j;
    v[j] = g < ng ? __builtin_nontemporal_load(&xr[g]) : u32x4{0u, 0u, 0u, 0u};
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < NR; ++j) a = amax8(v[j], a);
  const RowScale rs = row_scale(wave_max(a), scales, row, lane);
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int g = lane + 64 * j;
    if (g < ng) __builtin_nontemporal_store(encode8(v[j], rs.s, rs.r, rs.corrected), &cr[g]);
  }
}

// One row per 256-thread workgroup, at most 256 * 8 * NR elements, held in registers.
template <int NR>
__global__ void __launch_bounds__(256) fp8r_quantize_block_kernel(const u32x4* __restrict__ x,
                                                                  int64_t K,
                                                                  u32x2* __restrict__ codes,
                                                                  float* __restrict__ scales) {
  __shared__ float wmax[4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int64_t row = blockIdx.x;
  const int ng = (int)(K >> 3);
  const u32x4* xr = x + row * ng;
  u32x2* cr = codes + row * ng;
  u32x4 v[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int g = t + 256 * j;
    v[j] = g < ng ? __builtin_nontemporal_load(&xr[g]) : u32x4{0u, 0u, 0u, 0u};
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < NR; ++j) a = amax8(v[j], a);
  a = wave_max(a);
  if (lane == 0) wmax[t >> 6] = a;
  __syncthreads();
  a = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
  const RowScale rs = row_scale(a, scales, row, t);
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int g = t + 256 * j;
    if (g < ng) __builtin_nontemporal_store(encode8(v[j], rs.s, rs.r, rs.corrected), &cr[g]);
  }
}

template <int UNROLL>
__global__ void __launch_bounds__(256) fp8r_quantize_kernel(const u32x4* __restrict__ x,
                                                            int64_t M, int64_t K,
                                                            u32x2* __restrict__ codes,
                                                            float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves
  const int64_t ng = K >> 3;  // 8-element groups of the row
  const u32x4* xr = x + row * ng;
  u32x2* cr = codes + row * ng;

  float a = 0.0f;
  for (int64_t g0 = lane; g0 < ng; g0 += 64 * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t g = g0 + 64 * u;
      v[u] = g < ng ? xr[g] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) a = amax8(v[u], a);
  }
  const RowScale rs = row_scale(wave_max(a), scales, row, lane);
  for (int64_t g0 = lane; g0 < ng; g0 += 64 * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t g = g0 + 64 * u;
      v[u] = g < ng ? xr[g] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t g = g0 + 64 * u;
      if (g < ng) cr[g] = encode8(v[u], rs.s, rs.r, rs.corrected);
    }
  }
}

}  // namespace

hipError_t launch_fp8r_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                                hipStream_t stream, const LaunchInfo& dev) {
  (void)dev;
  if (M == 0) return hipSuccess;
  constexpr int kRowsPerBlock = 4;
  const int64_t blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * kRowsPerBlock);
  const u32x4* xv = (const u32x4*)x;
  u32x2* cv = (u32x2*)codes;
  float* sv = (float*)scales;
  const int64_t ng = K / 8;  // 16-byte loads per row
  if (ng <= 64 * 4) {  // one wave per row
    if (ng <= 64) hipLaunchKernelGGL((fp8r_quantize_regs_kernel<1>), grid, block, 0, stream, xv, M, K, cv, sv);
    else if (ng <= 128) hipLaunchKernelGGL((fp8r_quantize_regs_kernel<2>), grid, block, 0, stream, xv, M, K, cv, sv);
    else hipLaunchKernelGGL((fp8r_quantize_regs_kernel<4>), grid, block, 0, stream, xv, M, K, cv, sv);
  } else if (ng <= 256 * 8) {  // one workgroup per row
    if (M > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 rows((unsigned)M);
    if (ng <= 256 * 2) hipLaunchKernelGGL((fp8r_quantize_block_kernel<2>), rows, dim3(256), 0, stream, xv, K, cv, sv);
    else if (ng <= 256 * 4) hipLaunchKernelGGL((fp8r_quantize_block_kernel<4>), rows, dim3(256), 0, stream, xv, K, cv, sv);
    else if (ng <= 256 * 6) hipLaunchKernelGGL((fp8r_quantize_block_kernel<6>), rows, dim3(256), 0, stream, xv, K, cv, sv);
    else hipLaunchKernelGGL((fp8r_quantize_block_kernel<8>), rows, dim3(256), 0, stream, xv, K, cv, sv);
  } else {
    hipLaunchKernelGGL((fp8r_quantize_kernel<4>), grid, block, 0, stream, xv, M, K, cv, sv);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
