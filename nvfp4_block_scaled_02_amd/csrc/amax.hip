// Tensor amax for calibrating a global scale (the pages' calibrated fp32 input_scale and
// stored weight_scale_2, "BFL (fp8r / nvfp4)", nvfp4 item): max |x| over a bf16 tensor.
//
// Device-side calibration (launch_calibrate) adds a one-lane kernel that turns the amax
// into the global scale in place, so a dynamic scale never visits the host.
//
// Two launches on the caller's stream: a one-lane kernel clears the result, then a
// grid-stride kernel (two workgroups per CU) reduces four independent 16-byte loads per
// lane and step, reduces each wave with cross-lane moves and the workgroup through LDS,
// and merges workgroup results with one integer atomic max each on the fp32 bit pattern
// (non-negative binary32 values order like their bit patterns). Few atomics matter: they
// all hit one address. No memset is issued.
#include "codec.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

__global__ void clear_kernel(uint32_t* out) { *out = 0u; }

// In place: the amax (as fp32) becomes the global scale RN(amax / 2688) clamped into
// [2^-90, 2^90] (1 for amax == 0), the host's formula evaluated on the device.
__global__ void gs_from_amax_kernel(float* v) {
  const float a = *v;
  *v = a > 0.0f ? clamp_global_scale(a / 2688.0f) : 1.0f;
}

__device__ __forceinline__ uint32_t abs_max_bf16x2(uint32_t acc, uint32_t w) {
  // |lo| and |hi| as fp32 bit patterns; integer max is the fp32 max for these.
  const uint32_t lo = (w << 16) & 0x7FFF0000u;
  const uint32_t hi = w & 0x7FFF0000u;
  acc = acc > lo ? acc : lo;
  return acc > hi ? acc : hi;
}

__global__ void __launch_bounds__(256) amax_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                   const uint16_t* __restrict__ tail,
                                                   int64_t ntail, uint32_t* __restrict__ out) {
  constexpr int U = 4;
  __shared__ uint32_t wave_max[4];
  uint32_t m = 0u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < nvec; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&x[i + u * stride]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m = abs_max_bf16x2(m, v[u].x);
      m = abs_max_bf16x2(m, v[u].y);
      m = abs_max_bf16x2(m, v[u].z);
      m = abs_max_bf16x2(m, v[u].w);
    }
  }
  for (; i < nvec; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(&x[i]);
    m = abs_max_bf16x2(m, v.x);
    m = abs_max_bf16x2(m, v.y);
    m = abs_max_bf16x2(m, v.z);
    m = abs_max_bf16x2(m, v.w);
  }
  if (blockIdx.x == 0 && threadIdx.x < ntail) {
    const uint32_t t = ((uint32_t)tail[threadIdx.x] << 16) & 0x7FFF0000u;
    m = m > t ? m : t;
  }
  // wave reduction, then the workgroup's four waves through LDS
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
    m = m > o ? m : o;
  }
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = wave_max[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) w = w > wave_max[k] ? w : wave_max[k];
    if (w != 0u) atomicMax(out, w);
  }
}

}  // namespace

hipError_t launch_amax(const void* x, int64_t n, float* out, hipStream_t stream,
                       const LaunchInfo& dev) {
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, stream, (uint32_t*)out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  const int64_t nvec = n / 8;
  const int64_t ntail = n - nvec * 8;
  int64_t grid = (nvec + 1023) / 1024;
  const int64_t cap = (int64_t)dev.num_cus * 2;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const u32x4*)x,
                     nvec, (const uint16_t*)x + nvec * 8, ntail, (uint32_t*)out);
  return hipGetLastError();
}

hipError_t launch_calibrate(const void* x, int64_t n, float* gs, hipStream_t stream,
                            const LaunchInfo& dev) {
  hipError_t e = launch_amax(x, n, gs, stream, dev);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gs_from_amax_kernel, dim3(1), dim3(1), 0, stream, gs);
  return hipGetLastError();
}

}  // namespace nvfp4
