// Block-scaled W4A4 GEMM for gfx950: out[M, N] (bf16) = alpha * A_hat[M, K] W_hat[N, K]^T
// with A_hat, W_hat decoded from NVFP4 (E2M1 codes x per-16 E4M3 scales).
//
// This is the counterpart of the FP4 GEMM the pages pair with run-time activation
// quantization ("BFL (fp8r / nvfp4)", Kernels table, nvfp4 row); the pages state the
// workload suits high-batch, compute-bound runs (zubnet.ai page, paragraph 4), so the
// design targets the matrix cores.
//
// Why f16 MFMA: gfx950's block-scaled MFMA takes power-of-two scales per 32 elements,
// while NVFP4 has 3-mantissa-bit E4M3 scales per 16, which vary along K and cannot be
// factored out of the K sum. A decoded value q * s has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in f16 (normal range); the f16 MFMA then forms
// exact products and accumulates in fp32. Decoding to fp8 would round (E4M3 keeps 4
// bits), so f16 (2.5 PFLOP/s dense) is the fastest exact MFMA type.
//
// Structure:
//  * Packed 4-bit tiles and scale bytes stream from HBM into LDS (double-buffered);
//    decode happens in registers right before the MFMA, so LDS holds 4-bit data and its
//    traffic stays 4x below an f16-staged design.
//  * LDS layout of a packed tile: for every 32-row group and 64-element K chunk, 64
//    slots of 16 bytes in MFMA lane order (slot h*32 + r holds row r, bytes
//    [16h, 16h+16) of the chunk). A wave reads its operand fragment with one 16-byte
//    LDS load per lane at address lane*16: no bank conflicts.
//  * K mapping: lane half h of a fragment feeds the MFMA's K slots [8h, 8h+8) with
//    elements 32h + 8j .. 32h + 8j + 7 of the chunk on k-step j (j = 0..3). Both
//    operands use the same mapping, so each product pairs equal k; each lane's 8
//    elements sit inside one 16-element block and share one scale.
//  * Decode: the gfx950 conversion v_cvt_scalef32_pk_f16_fp4 turns two codes into two
//    f16 values, v_cvt_scalef32_pk_f16_fp8 turns a lane's two E4M3 scale bytes into f16,
//    and one packed f16 multiply per pair gives q * s exactly (all values are normal
//    f16, so no step depends on the denormal mode).
//  * The weights are the MFMA's A operand and the activations its B operand, so each
//    lane ends up holding 4 consecutive output columns of one row: 8-byte bf16 stores.
//  * Epilogue: fp32 accumulator * alpha (fp32), round to nearest even bf16.
#include "codec.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

constexpr int kThreads = 256;

template <int BM, int BN, int KC>
struct alignas(16) GemmSmem {
  uint8_t x[2][KC][BM * 32];   // activations, fragment order
  uint8_t w[2][KC][BN * 32];   // weights, fragment order
  uint32_t xs[2][KC][BM];      // 4 activation scale bytes per row and chunk
  uint32_t ws[2][KC][BN];      // 4 weight scale bytes per row and chunk
};

// Registers that carry one stage from global memory to LDS.
template <int ROWS, int KC>
struct StageRegs {
  static constexpr int kPieces = ROWS * KC * 2 / kThreads;  // 16-byte pieces per thread
  static constexpr int kScales = (ROWS * KC + kThreads - 1) / kThreads;
  static constexpr bool kScalesExact = (ROWS * KC) % kThreads == 0;
  u32x4 piece[kPieces];
  uint32_t scale[kScales];
};

// Load one operand's stage (ROWS rows starting at row0, K chunks [k64, k64 + KC)).
// kFast: K is a multiple of 64*KC and rows are 16-byte aligned (K % 32 == 0).
template <int ROWS, int KC, bool kFast>
__device__ __forceinline__ void load_stage(StageRegs<ROWS, KC>& r, const uint8_t* __restrict__ packed,
                                           const uint8_t* __restrict__ scales, int64_t row0,
                                           int64_t nrows, int64_t K, int64_t k64, int tid) {
  const int64_t pitch = K >> 1;
  const int64_t spitch = K >> 4;
#pragma unroll
  for (int p = 0; p < StageRegs<ROWS, KC>::kPieces; ++p) {
    const int i = tid + p * kThreads;
    const int row = i % ROWS;
    const int kh = i / ROWS;  // chunk * 2 + half
    int64_t grow = row0 + row;
    grow = grow < nrows ? grow : nrows - 1;
    const int64_t kel = (k64 + (kh >> 1)) * 64 + (kh & 1) * 32;  // first element of the piece
    const uint8_t* src = packed + grow * pitch + (kel >> 1);
    if constexpr (kFast) {
      r.piece[p] = *(const u32x4*)src;
    } else {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kel + 32 <= K) {
        const u32x2 a = *(const u32x2*)src;
        const u32x2 b = *(const u32x2*)(src + 8);
        v = u32x4{a.x, a.y, b.x, b.y};
      } else if (kel + 16 <= K) {
        const u32x2 a = *(const u32x2*)src;
        v = u32x4{a.x, a.y, 0u, 0u};
      }
      r.piece[p] = v;
    }
  }
#pragma unroll
  for (int q = 0; q < StageRegs<ROWS, KC>::kScales; ++q) {
    const int i = tid + q * kThreads;
    if (StageRegs<ROWS, KC>::kScalesExact || i < ROWS * KC) {
      const int row = i % ROWS;
      const int kc = i / ROWS;
      int64_t grow = row0 + row;
      grow = grow < nrows ? grow : nrows - 1;
      const int64_t blk = (k64 + kc) * 4;  // first scale of the chunk
      const uint8_t* src = scales + grow * spitch + blk;
      if constexpr (kFast) {
        r.scale[q] = *(const uint32_t*)src;
      } else {
        uint32_t v = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (blk + e < spitch) v |= (uint32_t)src[e] << (8 * e);
        r.scale[q] = v;
      }
    }
  }
}

template <int ROWS, int KC>
__device__ __forceinline__ void store_stage(const StageRegs<ROWS, KC>& r, uint8_t (*dst)[ROWS * 32],
                                            uint32_t (*dscale)[ROWS], int tid) {
#pragma unroll
  for (int p = 0; p < StageRegs<ROWS, KC>::kPieces; ++p) {
    const int i = tid + p * kThreads;
    const int row = i % ROWS;
    const int kh = i / ROWS;
    const int slot = (row >> 5) * 64 + (kh & 1) * 32 + (row & 31);
    *(u32x4*)&dst[kh >> 1][slot * 16] = r.piece[p];
  }
#pragma unroll
  for (int q = 0; q < StageRegs<ROWS, KC>::kScales; ++q) {
    const int i = tid + q * kThreads;
    if (StageRegs<ROWS, KC>::kScalesExact || i < ROWS * KC) dscale[i / ROWS][i % ROWS] = r.scale[q];
  }
}

template <int BM, int BN, int KC, bool kHw, bool kFast>
__global__ void __launch_bounds__(kThreads) gemm_kernel(GemmProblem p) {
  __shared__ GemmSmem<BM, BN, KC> sm;
  constexpr int WTM = BM / 2;  // activation rows per wave
  constexpr int WTN = BN / 2;  // weight rows (output columns) per wave
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_n = wave & 1;
  const int wave_m = wave >> 1;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tile_m = blockIdx.x / tiles_n;
  const int64_t tile_n = blockIdx.x % tiles_n;
  const int64_t m0 = tile_m * BM;
  const int64_t n0 = tile_n * BN;
  const int64_t nk = (p.K + 64 * KC - 1) / (64 * KC);

  floatx16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  StageRegs<BM, KC> xr;
  StageRegs<BN, KC> wr;
  load_stage<BM, KC, kFast>(xr, p.a_packed, p.a_scales, m0, p.M, p.K, 0, tid);
  load_stage<BN, KC, kFast>(wr, p.w_packed, p.w_scales, n0, p.N, p.K, 0, tid);
  store_stage<BM, KC>(xr, sm.x[0], sm.xs[0], tid);
  store_stage<BN, KC>(wr, sm.w[0], sm.ws[0], tid);
  __syncthreads();

  const int h = lane >> 5;
  const int r32 = lane & 31;

  for (int64_t t = 0; t < nk; ++t) {
    const int buf = (int)(t & 1);
    if (t + 1 < nk) {
      load_stage<BM, KC, kFast>(xr, p.a_packed, p.a_scales, m0, p.M, p.K, (t + 1) * KC, tid);
      load_stage<BN, KC, kFast>(wr, p.w_packed, p.w_scales, n0, p.N, p.K, (t + 1) * KC, tid);
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 wraw[FN], xraw[FM];
      uint32_t wsc[FN], xsc[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        wraw[i] = *(const u32x4*)&sm.w[buf][kc][((wave_n * FN + i) * 64 + lane) * 16];
        wsc[i] = *(const uint16_t*)((const uint8_t*)&sm.ws[buf][kc][wave_n * WTN + i * 32 + r32] + 2 * h);
      }
#pragma unroll
      for (int g = 0; g < FM; ++g) {
        xraw[g] = *(const u32x4*)&sm.x[buf][kc][((wave_m * FM + g) * 64 + lane) * 16];
        xsc[g] = *(const uint16_t*)((const uint8_t*)&sm.xs[buf][kc][wave_m * WTM + g * 32 + r32] + 2 * h);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8_t wf[FN], xf[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const half2_t s01 = scales_to_f16<kHw>(wsc[i]);
          wf[i] = decode8<kHw>(wraw[i][j], j < 2 ? s01.xx : s01.yy);
        }
#pragma unroll
        for (int g = 0; g < FM; ++g) {
          const half2_t s01 = scales_to_f16<kHw>(xsc[g]);
          xf[g] = decode8<kHw>(xraw[g][j], j < 2 ? s01.xx : s01.yy);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int g = 0; g < FM; ++g)
            acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], xf[g], acc[i][g], 0, 0, 0);
      }
    }
    if (t + 1 < nk) {
      store_stage<BM, KC>(xr, sm.x[buf ^ 1], sm.xs[buf ^ 1], tid);
      store_stage<BN, KC>(wr, sm.w[buf ^ 1], sm.ws[buf ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue: lane holds, for weight group i and activation group g, output row
  // m = m_base + r32 and columns n_base + 8q + 4h + {0..3} in acc[i][g][4q..4q+3].
  const bool n_vec = (p.N & 3) == 0;
#pragma unroll
  for (int g = 0; g < FM; ++g) {
    const int64_t m = m0 + wave_m * WTM + g * 32 + r32;
    if (m >= p.M) continue;
    uint16_t* orow = p.out + m * p.N;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wave_n * WTN + i * 32 + 8 * q + 4 * h;
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = bf16_rne(acc[i][g][4 * q + e] * p.alpha);
        if (n_vec && n + 3 < p.N) {
          *(u32x2*)&orow[n] = u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) orow[n + e] = (uint16_t)b[e];
        }
      }
    }
  }
}

template <int BM, int BN, int KC>
hipError_t launch_tile(const GemmProblem& p, hipStream_t stream, bool fast) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (fast)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, KC, true, true>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, KC, true, false>), dim3((unsigned)tiles), dim3(kThreads),
                       0, stream, p);
  return hipGetLastError();
}

// ---- decode self-test: the GEMM's decode on every (packed byte, scale) pair ----------

template <bool kHw>
__global__ void selftest_decode_kernel(const uint8_t* __restrict__ packed,
                                       const uint8_t* __restrict__ scales,
                                       uint16_t* __restrict__ out, int64_t nbytes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i * 4 >= nbytes) return;
  // four packed bytes (8 codes) and their (shared) scale code
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (i * 4 + e < nbytes) word |= (uint32_t)packed[i * 4 + e] << (8 * e);
  const half2_t s2 = scales_to_f16<kHw>(scales[i]);
  const half8_t v = decode8<kHw>(word, s2.xx);
  // Store the whole vector (the GEMM also consumes whole vectors): this compiler
  // version folds per-element reads of the fp4->f16 conversion result to its low
  // element, so no element is extracted here. nbytes is a multiple of 4.
  *(u32x4*)&out[i * 8] = __builtin_bit_cast(u32x4, v);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev) {
  (void)dev;
  const bool aligned = ((uintptr_t)p.a_packed % 16 == 0) && ((uintptr_t)p.w_packed % 16 == 0) &&
                       ((uintptr_t)p.a_scales % 4 == 0) && ((uintptr_t)p.w_scales % 4 == 0);
  constexpr int BM = 256, BN = 256, KC = 2;
  const bool fast = aligned && (p.K % (64 * KC) == 0);
  return launch_tile<BM, BN, KC>(p, stream, fast);
}

hipError_t launch_selftest_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* hw,
                                  uint16_t* sw, int64_t nbytes, hipStream_t stream) {
  if (nbytes == 0) return hipSuccess;
  if (nbytes % 4 != 0 || (uintptr_t)hw % 16 != 0 || (uintptr_t)sw % 16 != 0)
    return hipErrorInvalidValue;
  const int64_t nthreads = (nbytes + 3) / 4;
  const unsigned grid = (unsigned)((nthreads + 255) / 256);
  hipLaunchKernelGGL(selftest_decode_kernel<true>, dim3(grid), dim3(256), 0, stream, packed, scales,
                     hw, nbytes);
  hipLaunchKernelGGL(selftest_decode_kernel<false>, dim3(grid), dim3(256), 0, stream, packed, scales,
                     sw, nbytes);
  return hipGetLastError();
}

}  // namespace nvfp4
