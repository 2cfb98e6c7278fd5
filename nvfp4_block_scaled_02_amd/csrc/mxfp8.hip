// MXFP8 path for gfx950: quantize (bf16 -> E4M3 codes with one E8M0 scale per 32
// elements) and a GEMM on gfx950's block-scaled MFMA.
//
// MXFP8 is the second microscaling format the zubnet.ai page measures (paragraph 1): the
// Open Compute Project standard, 8-bit E4M3/E5M2 elements in 32-element blocks sharing
// one scale. This library takes E4M3 elements and the OCP E8M0 scale (a power of two,
// 2^(byte - 127)); the shared exponent of a block is floor(log2(amax)) - 8 (8 being the
// exponent of E4M3's largest normal, 448), clamped to [-127, 127], an all-zero block
// taking byte 0; elements are the E4M3 value nearest to x / 2^e, ties to even,
// saturating at 448, sign copied.
//
// Unlike NVFP4's E4M3-per-16 scales, these power-of-two per-32 scales are exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies, so the GEMM needs no decode: the fp8 codes go
// from HBM through LDS straight into the matrix core (fp8 rate, 2x the f16 rate).
#include "gemm_common.hpp"

namespace nvfp4 {

namespace {

__device__ __forceinline__ void mx_unpack_bf16x8(const u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = u2f(w[i] << 16);
    f[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
  }
}

// x / 2^e clamped to [-448, 448] (sign of zero kept): the conversion below then never
// overflows, and the clamp is the format's saturation.
__device__ __forceinline__ float mx_scaled(float x, int e) {
  return __builtin_fminf(__builtin_fmaxf(__builtin_ldexpf(x, -e), -kE4M3Max), kE4M3Max);
}

// Shared exponent of a block from its amax (>= 0): floor(log2(amax)) - 8 from the
// binary32 exponent field, clamped to [-127, 127]; zero and binary32-subnormal maxima
// (floor(log2) <= -127) give -127.
__device__ __forceinline__ int mx_shared_exponent(float amax) {
  const int eb = (int)(f2u(amax) >> 23);
  return eb == 0 ? -127 : max(eb - 135, -127);
}

// ---- quantize ----------------------------------------------------------------------
//
// Memory-bound: 2 B read, 1 + 1/32 B written per element. Four lanes share a 32-element
// block: lane 4i+q loads elements [8q, 8q+8) of block i (16 bytes, so a wave's load
// instruction reads 1 KiB of consecutive bytes), the block amax is the maximum over the
// quad (two DPP lane swaps), each lane converts its 8 elements with the gfx950 fp8
// conversion (round to nearest even; checked exhaustively against a software encoder by
// the self-test) and stores 8 code bytes; lane 4i writes the scale byte.
template <int UNROLL>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const u32x4* __restrict__ x,
                                                          u32x2* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          int64_t nlanes) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * UNROLL;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * UNROLL + threadIdx.x; base < nlanes;
       base += stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t li = base + (int64_t)u * blockDim.x;
      v[u] = li < nlanes ? __builtin_nontemporal_load(&x[li]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t li = base + (int64_t)u * blockDim.x;
      float f[8];
      mx_unpack_bf16x8(v[u], f);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(f[i]));
      // quad maximum: lanes 4i..4i+3 (DPP quad_perm [1,0,3,2], then [2,3,0,1])
      a = __builtin_fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false)));
      a = __builtin_fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0x4E, 0xF, 0xF, false)));
      const int e = mx_shared_exponent(a);
      uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(f[0], e), mx_scaled(f[1], e), 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(f[2], e), mx_scaled(f[3], e), w0, true);
      uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(f[4], e), mx_scaled(f[5], e), 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(f[6], e), mx_scaled(f[7], e), w1, true);
      if (li < nlanes) {
        __builtin_nontemporal_store(u32x2{w0, w1}, &codes[li]);
        if ((li & 3) == 0) scales[li >> 2] = (uint8_t)(e + 127);
      }
    }
  }
}

// ---- GEMM ----------------------------------------------------------------------------
//
// out[M, N] (bf16) = A_hat[M, K] W_hat[N, K]^T, A and W MXFP8. 256 x 256 tiles, 2 x 2
// waves of 128 x 128 (4 x 4 blocks of 32 x 32), v_mfma_scale_f32_32x32x64_f8f6f4 with
// weights as the A operand.
//
// Operand layout of that MFMA (measured on the device): over a 64-element K step, lane
// (h, r) = (lane / 32, lane % 32) of an operand fragment holds row r's elements
// [16h, 16h+16) of the step's first 32-element block in bytes 0-15 and the same range of
// the second block in bytes 16-31; byte 0 of its scale register is the E8M0 scale of row
// r, block h. Both operands use this mapping.
//
// Stage (64 elements of K) layout in LDS: per 32-row group, two 1 KiB pieces (block
// half 0 and 1) of 64 lane slots of 16 bytes, so a lane reads its fragment with two
// conflict-free 16-byte reads; per row, the 32-bit word of the 4 scale bytes (128
// elements) that contains the stage's two. Four stage buffers; loads (direct-to-LDS
// buffer loads, rows past M or N read as zero) are issued three stages ahead; at the end
// of stage t each wave waits for every load it issued before stage t (stage t+3's stay
// in flight) and the workgroup meets at a barrier, so stage t+1, whose fragments are read
// during stage t, is always complete.
template <int BM, int BN>
struct alignas(16) MxSmem {
  uint8_t x[4][BM * 64];
  uint8_t w[4][BN * 64];
  uint32_t xs[4][BM];
  uint32_t ws[4][BN];
};

typedef int v8i_t __attribute__((ext_vector_type(8)));

// Requires K % 128 == 0, 16-byte aligned codes, 4-byte aligned scales, and
// (rows + one tile) x K below 2^31 for both operands (32-bit buffer offsets).
template <int BM, int BN>
__global__ void __launch_bounds__(256) gemm_mx_kernel(GemmProblem p) {
  constexpr int NW = 4, WM = 2, WN = 2;
  __shared__ MxSmem<BM, BN> sm;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int kPa = 2 * BM / 32, kPw = 2 * BN / 32, kSa = BM / 64, kSw = BN / 64;
  static_assert(kPa % NW == 0 && kPw % NW == 0 && kSa % NW == 0 && kSw % NW == 0,
                "loads divide evenly among waves");
  constexpr int kPaW = kPa / NW, kPwW = kPw / NW, kSaW = kSa / NW, kSwW = kSw / NW;
  constexpr int kLoadsPerWave = kPaW + kPwW + kSaW + kSwW;
  static_assert(kLoadsPerWave < 16, "one stage of loads fits the vmcnt immediate");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_n = wave % WN;
  const int wave_m = wave / WN;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  int tile_m, tile_n;
  tile_order(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;
  const int nk = (int)(p.K / 64);
  const uint32_t pitch = (uint32_t)p.K;        // code bytes per row
  const uint32_t spitch = (uint32_t)(p.K >> 5);  // scale bytes per row

  const __amdgpu_buffer_rsrc_t rxp = make_rsrc(p.a_packed, (uint32_t)p.M * pitch);
  const __amdgpu_buffer_rsrc_t rwp = make_rsrc(p.w_packed, (uint32_t)p.N * pitch);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.a_scales, (uint32_t)p.M * spitch);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.w_scales, (uint32_t)p.N * spitch);
  const uint32_t voff_p = r32 * pitch + h * 16;
  const uint32_t voff_s = lane * spitch;

  // Load j of this wave for `stage` into buffer `buf` (lists: packed x, packed w,
  // scales x, scales w; wave w takes entries j' * NW + w of each).
  auto issue = [&](int j, int stage, int buf) {
    if (j < kPaW) {
      const int i = j * NW + wave, g = i >> 1, pc = i & 1;
      buffer_load_lds16(rxp, &sm.x[buf][g * 2048 + pc * 1024], voff_p,
                        (uint32_t)(m0 + 32 * g) * pitch + (uint32_t)stage * 64 + pc * 32);
    } else if (j < kPaW + kPwW) {
      const int i = (j - kPaW) * NW + wave, g = i >> 1, pc = i & 1;
      buffer_load_lds16(rwp, &sm.w[buf][g * 2048 + pc * 1024], voff_p,
                        (uint32_t)(n0 + 32 * g) * pitch + (uint32_t)stage * 64 + pc * 32);
    } else if (j < kPaW + kPwW + kSaW) {
      const int g = (j - kPaW - kPwW) * NW + wave;
      buffer_load_lds4(rxs, &sm.xs[buf][g * 64], voff_s,
                       (uint32_t)(m0 + 64 * g) * spitch + (uint32_t)(stage >> 1) * 4);
    } else {
      const int g = (j - kPaW - kPwW - kSaW) * NW + wave;
      buffer_load_lds4(rws, &sm.ws[buf][g * 64], voff_s,
                       (uint32_t)(n0 + 64 * g) * spitch + (uint32_t)(stage >> 1) * 4);
    }
  };

  floatx16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  // fragments and scale bytes of two stages (by parity)
  v8i_t wf[2][FN], xf[2][FM];
  int wsc[2][FN], xsc[2][FM];
  const int wfrag = wave_n * FN * 2048 + lane * 16;
  const int xfrag = wave_m * FM * 2048 + lane * 16;
  auto read_stage = [&](int par, int buf, int stage) {
    const int sb = (stage & 1) * 2 + h;  // byte of the scale word: block h of this stage
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const u32x4 a = *(const u32x4*)&sm.w[buf][wfrag + i * 2048];
      const u32x4 b = *(const u32x4*)&sm.w[buf][wfrag + i * 2048 + 1024];
      wf[par][i] = v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      wsc[par][i] = ((const uint8_t*)sm.ws[buf])[(wave_n * WTN + i * 32 + r32) * 4 + sb];
    }
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      const u32x4 a = *(const u32x4*)&sm.x[buf][xfrag + g * 2048];
      const u32x4 b = *(const u32x4*)&sm.x[buf][xfrag + g * 2048 + 1024];
      xf[par][g] = v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      xsc[par][g] = ((const uint8_t*)sm.xs[buf])[(wave_m * WTM + g * 32 + r32) * 4 + sb];
    }
  };

  // prologue: stages 0, 1 and 2 into buffers 0, 1 and 2, then read stage 0
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) issue(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) issue(j, nk > 1 ? 1 : nk - 1, 1);
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) issue(j, nk > 2 ? 2 : nk - 1, 2);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  read_stage(0, 0, 0);

  constexpr int kMfma = FN * FM;
  constexpr int kReads = 3 * (FN + FM);
  // One stage; `cur` (the register set of stage t's fragments) must be a constant, so
  // the loop below runs two stages per iteration.
  auto stage = [&](int t, int buf, const int cur) {
    const int nbuf = (buf + 1) & 3;  // stage t + 1
    const int lbuf = (buf + 3) & 3;  // stage t + 3 (its buffer held stage t - 1)
    const int lstage = t + 3 < nk ? t + 3 : nk - 1;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) issue(j, lstage, lbuf);
    read_stage(cur ^ 1, nbuf, t + 1 < nk ? t + 1 : t);
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int g = 0; g < FM; ++g)
        acc[i][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0, wsc[cur][i], 0, xsc[cur][g]);
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (q < kLoadsPerWave) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS
      if (q * 2 < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU (fragment moves)
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kLoadsPerWave>();
    __builtin_amdgcn_s_barrier();
  };
  int buf = 0;
  for (int t = 0; t < nk; t += 2) {  // nk is even (K % 128 == 0)
    stage(t, buf, 0);
    stage(t + 1, (buf + 1) & 3, 1);
    buf = (buf + 2) & 3;
  }

  // drain the last (unused) loads before the stage buffers stage the stores
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  static_assert(NW * 32 * FN * 32 * 2 <= sizeof(sm.x), "store staging fits");
  store_tile_lds<FM, FN>(acc, p, (int64_t)m0 + wave_m * WTM, (int64_t)n0 + wave_n * WTN, lane,
                         (uint16_t*)&sm.x[0][0] + wave * 32 * FN * 32);
}

// ---- self-test: the fp8 conversion against the software E4M3 encoder ----------------

// Every binary32 pattern except NaN and Inf: y clamped to [-448, 448] as the quantizer
// does, converted by the hardware, and encoded by the software encoder (sign of y, then
// nearest E4M3 magnitude with ties to even, saturating at 448).
__global__ void mx_selftest_e4m3_exhaustive_kernel(unsigned long long* __restrict__ count,
                                                   uint32_t* __restrict__ first) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t nthreads = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u = tid; u < (1ull << 32); u += nthreads) {
    const uint32_t bits = (uint32_t)u;
    if (((bits >> 23) & 0xFFu) == 0xFFu) continue;
    const float y = __builtin_fminf(__builtin_fmaxf(u2f(bits), -kE4M3Max), kE4M3Max);
    const uint32_t hw = __builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu;
    const uint32_t sw = ((bits >> 31) << 7) | e4m3_encode_sat(__builtin_fabsf(y));
    if (hw != sw) {
      const unsigned long long k = atomicAdd(count, 1ull);
      if (k < 16) first[k] = bits;
    }
  }
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                              hipStream_t stream, const LaunchInfo& dev) {
  const int64_t nlanes = M * K / 8;
  if (nlanes == 0) return hipSuccess;
  constexpr int kThreads = 256, kUnroll = 2;
  const int64_t want = (nlanes + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  const int64_t cap = (int64_t)dev.num_cus * 32;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL((mx_quantize_kernel<kUnroll>), dim3(grid), dim3(kThreads), 0, stream,
                     (const u32x4*)x, (u32x2*)codes, (uint8_t*)scales, nlanes);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev) {
  (void)dev;
  constexpr int BM = 256, BN = 256;
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_mx_kernel<BM, BN>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_mx_selftest_e4m3_exhaustive(unsigned long long* count, uint32_t* first,
                                              hipStream_t stream) {
  hipLaunchKernelGGL(mx_selftest_e4m3_exhaustive_kernel, dim3(8192), dim3(256), 0, stream, count,
                     first);
  return hipGetLastError();
}

}  // namespace nvfp4
