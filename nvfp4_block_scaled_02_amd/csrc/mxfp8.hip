// MXFP8 path for gfx950: quantize (bf16 -> E4M3 or E5M2 codes with one E8M0 scale per
// 32 elements) and a GEMM on gfx950's block-scaled MFMA.
//
// MXFP8 is the second microscaling format the zubnet.ai page measures (paragraph 1): the
// Open Compute Project standard, 8-bit E4M3/E5M2 elements in 32-element blocks sharing
// one scale. This library takes either element type with the OCP E8M0 scale (a power of
// two, 2^(byte - 127)); the shared exponent of a block is floor(log2(amax)) - emax (emax
// the exponent of the element type's largest normal: 8 for E4M3's 448, 15 for E5M2's
// 57344), clamped to [-127, 127], an all-zero block taking byte 0; elements are the
// value of the element type nearest to x / 2^e, ties to even, saturating at its largest
// finite value, sign copied. The GEMM takes each operand's element type separately (the
// MFMA's operand format fields).
//
// Unlike NVFP4's E4M3-per-16 scales, these power-of-two per-32 scales are exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies, so the GEMM needs no decode: the fp8 codes go
// from HBM through LDS straight into the matrix core (fp8 rate, 2x the f16 rate).
//
// The same GEMM kernels, with unit block scales and a per-row x per-column scale
// epilogue, run the rowwise FP8 ("fp8r") product; its quantizer is in fp8r.hip.
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

// x / 2^e clamped to the element type's finite range, [-448, 448] or [-57344, 57344]
// (sign of zero kept): the conversion below then never overflows, and the clamp is the
// format's saturation.
template <bool kE5M2>
__device__ __forceinline__ float mx_scaled(float x, int e) {
  constexpr float lim = kE5M2 ? kE5M2Max : kE4M3Max;
  return __builtin_fminf(__builtin_fmaxf(__builtin_ldexpf(x, -e), -lim), lim);
}

// Shared exponent of a block from its amax (>= 0): floor(log2(amax)) - emax (8 for E4M3,
// 15 for E5M2) from the binary32 exponent field, clamped to [-127, 127]; zero and
// binary32-subnormal maxima (floor(log2) <= -127) give -127.
template <bool kE5M2>
__device__ __forceinline__ int mx_shared_exponent(float amax) {
  const int eb = (int)(f2u(amax) >> 23);
  return eb == 0 ? -127 : max(eb - (kE5M2 ? 142 : 135), -127);
}

// Four elements y0..y3 (already scaled and clamped) into the element type's bytes
// 0..3 of a word (round to nearest even).
template <bool kE5M2>
__device__ __forceinline__ uint32_t mx_convert4(float y0, float y1, float y2, float y3) {
  if constexpr (kE5M2) {
    const uint32_t w = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
    return __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, w, true);
  } else {
    const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  }
}

// ---- quantize ----------------------------------------------------------------------
//
// Memory-bound: 2 B read, 1 + 1/32 B written per element. Four lanes share a 32-element
// block: lane 4i+q loads elements [8q, 8q+8) of block i (16 bytes, so a wave's load
// instruction reads 1 KiB of consecutive bytes), the block amax is the maximum over the
// quad (two DPP lane swaps), each lane converts its 8 elements with the gfx950 fp8
// conversion (round to nearest even; checked exhaustively against a software encoder by
// the self-test) and stores 8 code bytes; lane 4i writes the scale byte.
template <int UNROLL, bool kE5M2>
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
      const int e = mx_shared_exponent<kE5M2>(a);
      const uint32_t w0 = mx_convert4<kE5M2>(mx_scaled<kE5M2>(f[0], e), mx_scaled<kE5M2>(f[1], e),
                                             mx_scaled<kE5M2>(f[2], e), mx_scaled<kE5M2>(f[3], e));
      const uint32_t w1 = mx_convert4<kE5M2>(mx_scaled<kE5M2>(f[4], e), mx_scaled<kE5M2>(f[5], e),
                                             mx_scaled<kE5M2>(f[6], e), mx_scaled<kE5M2>(f[7], e));
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
// weights as the A operand. kFw and kFx are that MFMA's operand format codes for the
// weights (its A operand) and the activations (its B operand): 0 for E4M3, 1 for E5M2;
// both 8-bit types share the operand layout below.
//
// Operand layout of that MFMA (measured on the device): over a 64-element K step, lane
// (h, r) = (lane / 32, lane % 32) of an operand fragment holds row r's elements
// [16h, 16h+16) of the step's first 32-element block in bytes 0-15 and the same range of
// the second block in bytes 16-31; byte 0 of its scale register is the E8M0 scale of row
// r, block h. Both operands use this mapping.
//
// Loads. The direct-to-LDS path costs by the cache lines an instruction touches rather
// than by its bytes, so every load reads whole 64-byte row segments: a code load takes
// 16 rows x the stage's 64 bytes (4 lanes per row), a scale load 64 rows x 16 bytes (the
// scales of 512 elements, 8 stages), issued once every 8 stages. Rows past M or N read as
// zero (buffer range checks over row windows, window_rsrc).
//
// Stage (64 elements of K) layout in LDS: each 16-row piece is 1 KiB, row r's 64 bytes at
// 64 r, its 16-byte chunk c stored at slot c ^ chunk_swz(r) so that the fragment reads (two
// 16-byte reads per lane and block, chunks h and h + 2 of row r) hit distinct banks. Four
// code buffers, filled three stages ahead; two scale buffers of 8 stages, filled 8 stages
// ahead. At the end of stage t each wave waits for every load it issued before stage t
// and the workgroup meets at a barrier, so stage t+1, whose fragments are read during
// stage t, is always complete.
//
// Each stage issues its MFMAs, loads and LDS reads in one fixed interleaved order (one
// load and one or two reads after each MFMA) so that the matrix core never waits behind a
// burst of memory instructions.
template <int BM, int BN>
struct alignas(16) MxSmem {
  uint8_t x[4][BM * 64];
  uint8_t w[4][BN * 64];
  uint8_t xs[2][BM * 16];
  uint8_t ws[2][BN * 16];
};

typedef int v8i_t __attribute__((ext_vector_type(8)));

// Requires K % 128 == 0, 16-byte aligned codes, 4-byte aligned scales, and
// (rows + one tile) x K below 2^31 for both operands (32-bit buffer offsets).
//
// kRowwise: the rowwise FP8 product of the "BFL (fp8r / nvfp4)" page (fp8r item and
// Kernels table row: E4M3 operands with one fp32 scale per row). The per-row scales leave
// the K-sum, so the MFMA runs with unit block scales (E8M0 127, no scale loads) and the
// epilogue multiplies each output by a_scales[m] * w_scales[n] (fp32 arrays).
template <int BM, int BN, bool kRowwise, int kFw, int kFx>
__global__ void __launch_bounds__(256) gemm_mx_kernel(GemmProblem p) {
  constexpr int NW = 4, WM = 2, WN = 2;
  __shared__ MxSmem<BM, BN> sm;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int kPa = BM / 16, kPw = BN / 16;  // 1 KiB code pieces per stage
  constexpr int kSa = BM / 64, kSw = BN / 64;  // 1 KiB scale pieces per 8 stages
  static_assert(kPa % NW == 0 && kPw % NW == 0 && kSa % NW == 0 && kSw % NW == 0,
                "loads divide evenly among waves");
  constexpr int kPaW = kPa / NW, kPwW = kPw / NW;
  constexpr int kLoads = kPaW + kPwW;          // code loads per wave per stage
  constexpr int kSLoads = kRowwise ? 0 : (kSa + kSw) / NW;  // scale loads per wave per 8 stages
  constexpr int kMfma = FN * FM;
  static_assert(kLoads + kSLoads <= kMfma, "at most one load after each MFMA");
  static_assert(kLoads + kSLoads < 64, "one stage of loads fits the vmcnt counter");

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
  const int ngrp = (nk + 7) >> 3;                 // groups of 8 stages
  const uint32_t pitch = (uint32_t)p.K;          // code bytes per row
  const uint32_t spitch = (uint32_t)(p.K >> 5);  // scale bytes per row

  // row windows [m0, M) and [n0, N) (see window_rsrc): rows past M or N read as zero
  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, m0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, m0, p.M, spitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);

  // Code load j of this wave for `stage` into buffer `buf`: piece j * NW + wave of the
  // list (x pieces, then w pieces).
  auto issue_codes = [&](int j, int stage, int buf) {
    if (j < kPaW) {
      const int i = j * NW + wave;
      buffer_load_lds16(rxp, &sm.x[buf][i * 1024], code_piece_voff(lane, 16 * i, pitch),
                        (uint32_t)stage * 64);
    } else {
      const int i = (j - kPaW) * NW + wave;
      buffer_load_lds16(rwp, &sm.w[buf][i * 1024], code_piece_voff(lane, 16 * i, pitch),
                        (uint32_t)stage * 64);
    }
  };
  // Scale load j of this wave for stage group `grp` into scale buffer `sbuf` (a partial
  // last group reads past the row's end: that position is range-checked too).
  auto issue_scales = [&](int j, int grp, int sbuf) {
    if (j < kSa / NW) {
      const int i = j * NW + wave;
      buffer_load_lds16(rxs, &sm.xs[sbuf][i * 1024],
                        scale_piece_voff(lane, 64 * i, spitch, (uint32_t)grp * 16), 0);
    } else {
      const int i = (j - kSa / NW) * NW + wave;
      buffer_load_lds16(rws, &sm.ws[sbuf][i * 1024],
                        scale_piece_voff(lane, 64 * i, spitch, (uint32_t)grp * 16), 0);
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
  // lane's first 16-byte chunk within a 32-row group (2 KiB); the second is 32 bytes over
  const int fr0 = (r32 >> 4) * 1024 + (r32 & 15) * 64 + 16 * (h ^ chunk_swz(r32 & 15));
  const int fr1 = fr0 ^ 32;
  // LDS reads of one stage in the order its MFMAs need them: w0, x0..x(FM-1), w1, ...
  // Read k (of kReads) is a fragment half or a scale byte.
  constexpr int kReads = 3 * (FN + FM);
  auto read_one = [&](int k, int par, int buf, int stage) {
    const int sbuf = (stage >> 3) & 1;
    const int sbyte = (stage & 7) * 2 + h;
    const int f = k / 3, part = k % 3;  // operand fragment f: w0, x0, x1, .., w1, w2, ..
    const bool is_w = f == 0 || f > FM;
    const int idx = f == 0 ? 0 : (f <= FM ? f - 1 : f - FM);
    if (is_w) {
      const uint8_t* base = &sm.w[buf][(wave_n * FN + idx) * 2048];
      if (part == 0) {
        const u32x4 a = *(const u32x4*)&base[fr0];
        wf[par][idx][0] = (int)a.x; wf[par][idx][1] = (int)a.y; wf[par][idx][2] = (int)a.z; wf[par][idx][3] = (int)a.w;
      } else if (part == 1) {
        const u32x4 b = *(const u32x4*)&base[fr1];
        wf[par][idx][4] = (int)b.x; wf[par][idx][5] = (int)b.y; wf[par][idx][6] = (int)b.z; wf[par][idx][7] = (int)b.w;
      } else if (!kRowwise) {
        wsc[par][idx] = sm.ws[sbuf][(wave_n * WTN + idx * 32 + r32) * 16 + sbyte];
      }
    } else {
      const uint8_t* base = &sm.x[buf][(wave_m * FM + idx) * 2048];
      if (part == 0) {
        const u32x4 a = *(const u32x4*)&base[fr0];
        xf[par][idx][0] = (int)a.x; xf[par][idx][1] = (int)a.y; xf[par][idx][2] = (int)a.z; xf[par][idx][3] = (int)a.w;
      } else if (part == 1) {
        const u32x4 b = *(const u32x4*)&base[fr1];
        xf[par][idx][4] = (int)b.x; xf[par][idx][5] = (int)b.y; xf[par][idx][6] = (int)b.z; xf[par][idx][7] = (int)b.w;
      } else if (!kRowwise) {
        xsc[par][idx] = sm.xs[sbuf][(wave_m * WTM + idx * 32 + r32) * 16 + sbyte];
      }
    }
  };

  // prologue: scales of stages 0-7, codes of stages 0, 1 and 2, then read stage 0
#pragma unroll
  for (int j = 0; j < kSLoads; ++j) issue_scales(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue_codes(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue_codes(j, nk > 1 ? 1 : nk - 1, 1);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue_codes(j, nk > 2 ? 2 : nk - 1, 2);
  // scales and stages 0 and 1 (stage 0 reads stage 1's fragments ahead); stage 2's loads
  // may still be in flight: the wait at the end of stage 0 covers them
  wait_vmcnt<kLoads>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int k = 0; k < kReads; ++k) read_one(k, 0, 0, 0);

  // One stage. `cur` (the register set of stage t's fragments) and `sload` (t % 8 == 0
  // and a later stage group exists: load its scales into the other scale buffer) must be
  // constants, so that the stage is one basic block whose order the scheduling barriers
  // fix; the main loop runs 8 stages per iteration.
  auto stage = [&](int t, int buf, const int cur, const bool sload) {
    const int nbuf = (buf + 1) & 3;  // stage t + 1
    const int lbuf = (buf + 3) & 3;  // stage t + 3 (its buffer held stage t - 1)
    const int lstage = t + 3 < nk ? t + 3 : nk - 1;
    const int rstage = t + 1 < nk ? t + 1 : t;
    const int sgrp = (t >> 3) + 1 < ngrp ? (t >> 3) + 1 : ngrp - 1;
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      const int i = q / FM, g = q % FM;
      acc[i][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          wf[cur][i], xf[cur][g], acc[i][g], kFw, kFx, 0, kRowwise ? 127 : wsc[cur][i], 0,
          kRowwise ? 127 : xsc[cur][g]);
      if (q < kLoads) issue_codes(q, lstage, lbuf);
      else if (q < kLoads + kSLoads && sload) issue_scales(q - kLoads, sgrp, ((t >> 3) + 1) & 1);
#pragma unroll
      for (int k = q * kReads / kMfma; k < (q + 1) * kReads / kMfma; ++k) read_one(k, cur ^ 1, nbuf, rstage);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (sload) wait_vmcnt<kLoads + kSLoads>();
    else wait_vmcnt<kLoads>();
    __builtin_amdgcn_s_barrier();
  };
  // 8 stages per iteration (the code buffers cycle back to 0), then the last nk % 8
  // stages two at a time (nk is even: K % 128 == 0); their scales were loaded with the
  // group before, so they load none.
  int t = 0;
  for (; t + 8 <= nk; t += 8) {
    stage(t, 0, 0, true);
#pragma unroll
    for (int u = 1; u < 8; ++u) stage(t + u, u & 3, u & 1, false);
  }
  for (; t < nk; t += 2) {
    stage(t, t & 3, 0, false);
    stage(t + 1, (t + 1) & 3, 1, false);
  }

  // drain the last (unused) loads before the stage buffers stage the stores
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  store_tile_lds<FM, FN, kRowwise>(acc, p, Alpha{p.alpha, 0}, (int64_t)m0 + wave_m * WTM,
                                   (int64_t)n0 + wave_n * WTN, lane,
                                   (uint16_t*)&sm.x[0][0] + wave * 32 * kStoreRowPad(FN));
}

// ---- GEMM, 288 x 192 tiles ---------------------------------------------------------------
//
// The same product on 288 x 192 tiles: 4608 = 16 x 288 and every FLUX width (3072, 9216,
// 12288) is a multiple of 192, so these products split into whole multiples of 256 tiles
// (the 256 x 256 tile gives 216 tiles on 256 compute units for 4608 x 3072). The tile is
// 9 x 6 blocks of 32 x 32; wave (m, n) owns weight groups 3n..3n+2 and activation groups
// 0..3 (m = 0) or 5..8 (m = 1), and the middle activation group 4 is split by weight
// block: wave (0, n) takes its blocks with weight groups 3n and 3n+1, wave (1, n) the one
// with 3n+2. So the waves issue 14 and 13 MFMAs per stage (the 256 x 256 tile: 16) and no
// partial sums need to meet.
//
// The codes are loaded two stages (128 elements of K, a whole 128-byte line per row) at a
// time: each load fills 8 rows x 128 bytes (eight lanes per row), where the 256 x 256
// kernel's loads fill 16 rows x 64 bytes. Direct-to-LDS loads cost by the cache lines
// they touch, and this halves the lines per byte (measured on the device: 88.6 against
// 51.3 GB/s per compute unit of L2-resident data). LDS: two double-stage buffers (the bytes of four single stages), each row's 128
// bytes as eight 16-byte chunks at slots c ^ x_swz(row % 32), so the fragment reads (lane
// (h, r) of stage s reads chunks 4s + h and 4s + 2 + h of row r) hit distinct banks.
//
// Pipeline over double stages d (stages 2d, 2d+1, buffer d & 1):
//  * even stage 2d: MFMAs on stage 2d's fragments while stage 2d+1's are read (same
//    buffer); every 8 stages, the next scale group's loads;
//  * odd stage 2d+1: half of its MFMAs, then the wave waits for all its loads (those of
//    double stage d+1, issued during stage 2d-1) with its LDS reads landed and meets the
//    workgroup at a barrier; then, under the other MFMAs, it issues the loads of double
//    stage d+2 into buffer d & 1 (whose last fragments, stage 2d+1's, every wave read
//    during stage 2d) and reads stage 2d+2's fragments from buffer (d+1) & 1.
// So a load has about two stages of lead and LDS reads never wait at a stage boundary.
// The barrier's place in the odd stage (after NVFP4_MX_FIT_HALF of its MFMAs) was swept:
// 1 to 4 alike, later ones slower (4608 x 3072 x 12288: 130 us at 4, 135 at 7, 141 at 11).
#ifndef NVFP4_MX_FIT_HALF
#define NVFP4_MX_FIT_HALF 4
#endif

template <int BM, int BN>
struct alignas(16) MxFitSmem {
  static constexpr int kScaleRowsX = (BM + 63) / 64 * 64;
  uint8_t x[2][BM * 128];
  uint8_t w[2][BN * 128];
  uint8_t sc[2][(kScaleRowsX + BN) * 16];
};

template <int BM, int BN, bool kRowwise, int kS, int kFw, int kFx>
__device__ __forceinline__ void mx_fit_wave(const GemmProblem& p, MxFitSmem<BM, BN>& sm, int lane,
                                             int wave, int m0, int n0) {
  constexpr int NW = 4;
  constexpr int GX = BM / 32, GW = BN / 32;
  static_assert(GX * 32 == BM && GW * 32 == BN && GX % 2 == 1 && GW % 2 == 0, "fit tile shape");
  constexpr int FM = GX / 2;  // whole activation groups per wave
  constexpr int FN = GW / 2;  // weight groups per wave
  constexpr int GS = FM;      // the middle activation group
  constexpr int kI0 = kS == FN - 1 ? 0 : FN - kS;  // first weight block of the middle group
  constexpr int kPx = BM / 8, kPw = BN / 8;        // 1 KiB pieces per double stage
  static_assert((kPx + kPw) % NW == 0, "code pieces divide among waves");
  constexpr int kCode = (kPx + kPw) / NW;
  constexpr int kRowsSx = MxFitSmem<BM, BN>::kScaleRowsX;
  constexpr int kSx = kRowsSx / 64;
  static_assert(BN % 64 == 0 && (kSx + BN / 64) % NW == 0, "scale pieces divide among waves");
  constexpr int kSLoads = kRowwise ? 0 : (kSx + BN / 64) / NW;
  constexpr int kMfma = FN * FM + kS;
  constexpr int kHalf = NVFP4_MX_FIT_HALF;       // MFMAs of an odd stage before its barrier
  static_assert(kHalf < kMfma, "the barrier sits inside the odd stage");
  constexpr int kFrags = FN + FM + 1;
  constexpr int kReads = 3 * kFrags;             // fragment halves and scale bytes per stage
  constexpr int kTail = kMfma - kHalf;
  constexpr int kCodePer = (kCode + kTail - 1) / kTail;

  const int wave_n = wave & 1;
  const int wave_m = wave >> 1;
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const int nk = (int)(p.K / 64);  // stages (even: K % 128 == 0)
  const int nd = nk >> 1;          // double stages
  const int ngrp = (nk + 7) >> 3;  // scale groups of 8 stages
  const uint32_t pitch = (uint32_t)p.K;
  const uint32_t spitch = (uint32_t)(p.K >> 5);

  // row windows [m0, M) and [n0, N) (see window_rsrc)
  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, m0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, m0, p.M, spitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);

  // code piece j * NW + wave of double stage ds into buffer buf: activation pieces
  // (rows 8i .. 8i+7), then weight pieces
  auto issue_code = [&](int j, int ds, int buf) {
    const int i = j * NW + wave;
    if (i < kPx)
      buffer_load_lds16(rxp, &sm.x[buf][i * 1024], x_piece_voff(lane, 8 * i, pitch), (uint32_t)ds * 128);
    else
      buffer_load_lds16(rwp, &sm.w[buf][(i - kPx) * 1024], x_piece_voff(lane, 8 * (i - kPx), pitch),
                        (uint32_t)ds * 128);
  };
  // scale piece j * NW + wave (64 rows x 16 bytes): activation rows first, then weight rows
  auto issue_scales = [&](int j, int grp, int sbuf) {
    const int i = j * NW + wave;
    const bool isx = i < kSx;
    const int prow = isx ? 64 * i : 64 * (i - kSx);
    buffer_load_lds16(isx ? rxs : rws, &sm.sc[sbuf][i * 1024],
                      scale_piece_voff(lane, prow, spitch, (uint32_t)grp * 16), 0);
  };

  floatx16 acc[FN][FM], accs[kS];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;
#pragma unroll
  for (int s = 0; s < kS; ++s)
#pragma unroll
    for (int v = 0; v < 16; ++v) accs[s][v] = 0.0f;

  v8i_t wf[2][FN], xf[2][FM + 1];
  int wsc[2][FN], xsc[2][FM + 1];
  const int rbase = (r32 >> 3) * 1024 + (r32 & 7) * 128;  // lane's row within a 32-row group
  const int sw = x_swz(r32);
  const int xg0 = wave_m ? GS + 1 : 0;
  // read k of a stage (st: its index, for the buffer half and the scale byte): fragment
  // halves in the order the MFMAs need them (w0, x0..x(FM-1), w1, .., the middle group
  // last), each followed by its scale byte
  auto read_one = [&](int k, int par, int buf, int st) {
    const int sbuf = (st >> 3) & 1;
    const int sbyte = (st & 7) * 2 + h;
    const int f = k / 3, part = k % 3;
    const bool is_w = f == 0 || (f > FM && f < kFrags - 1);
    const int idx = f == 0 ? 0 : (f <= FM ? f - 1 : (f < kFrags - 1 ? f - FM : FM));
    const int grp = is_w ? wave_n * FN + idx : (idx < FM ? xg0 + idx : GS);
    if (part < 2) {
      const int chunk = 4 * (st & 1) + 2 * part + h;
      const uint8_t* base = is_w ? &sm.w[buf][grp * 4096] : &sm.x[buf][grp * 4096];
      const u32x4 a = *(const u32x4*)&base[rbase + 16 * (chunk ^ sw)];
      const int o = 4 * part;
      if (is_w) {
        wf[par][idx][o] = (int)a.x; wf[par][idx][o + 1] = (int)a.y;
        wf[par][idx][o + 2] = (int)a.z; wf[par][idx][o + 3] = (int)a.w;
      } else {
        xf[par][idx][o] = (int)a.x; xf[par][idx][o + 1] = (int)a.y;
        xf[par][idx][o + 2] = (int)a.z; xf[par][idx][o + 3] = (int)a.w;
      }
    } else if (!kRowwise) {
      const int row = is_w ? kRowsSx + grp * 32 + r32 : grp * 32 + r32;
      const int v = sm.sc[sbuf][row * 16 + sbyte];
      if (is_w) wsc[par][idx] = v;
      else xsc[par][idx] = v;
    }
  };
  auto mfma = [&](int q, int cur) {
    if (q < FN * FM) {
      const int i = q / FM, g = q % FM;
      acc[i][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          wf[cur][i], xf[cur][g], acc[i][g], kFw, kFx, 0, kRowwise ? 127 : wsc[cur][i], 0,
          kRowwise ? 127 : xsc[cur][g]);
    } else {
      const int sidx = q - FN * FM, i = kI0 + sidx;
      accs[sidx] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          wf[cur][i], xf[cur][FM], accs[sidx], kFw, kFx, 0, kRowwise ? 127 : wsc[cur][i], 0,
          kRowwise ? 127 : xsc[cur][FM]);
    }
  };

  // prologue: scales of group 0 and double stage 0, wait, then double stage 1's loads
  // (a double stage past the last reloads the last one into the free buffer) and stage
  // 0's fragments
#pragma unroll
  for (int j = 0; j < kSLoads; ++j) issue_scales(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kCode; ++j) issue_code(j, 0, 0);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int j = 0; j < kCode; ++j) issue_code(j, nd > 1 ? 1 : 0, 1);
#pragma unroll
  for (int k = 0; k < kReads; ++k) read_one(k, 0, 0, 0);

  // double stage d in buffer buf (a constant); sload: d % 4 == 0, so stage 2d starts a
  // scale group and the next group's scales load during it
  auto dstage = [&](int d, const int buf, const bool sload) {
    const int t0 = 2 * d;
    const int sgrp = (t0 >> 3) + 1 < ngrp ? (t0 >> 3) + 1 : ngrp - 1;
    // even stage: stage t0 + 1's fragments from the same buffer
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      mfma(q, 0);
      if (sload && q < kSLoads) issue_scales(q, sgrp, ((t0 >> 3) + 1) & 1);
#pragma unroll
      for (int k = q * kReads / kMfma; k < (q + 1) * kReads / kMfma; ++k) read_one(k, 1, buf, t0 + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // odd stage: first part, then every load of double stage d + 1 landed and the barrier
#pragma unroll
    for (int q = 0; q < kHalf; ++q) {
      mfma(q, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    const int lds_ = d + 2 < nd ? d + 2 : nd - 1;  // double stage loaded into buf
#pragma unroll
    for (int q = kHalf; q < kMfma; ++q) {
      mfma(q, 1);
      const int u = q - kHalf;
#pragma unroll
      for (int l = 0; l < kCodePer; ++l)
        if (u * kCodePer + l < kCode) issue_code(u * kCodePer + l, lds_, buf);
      // (after the last double stage these reads fetch bytes nothing uses: reading
      // unconditionally keeps the previous fragments from staying live)
#pragma unroll
      for (int k = u * kReads / kTail; k < (u + 1) * kReads / kTail; ++k) read_one(k, 0, buf ^ 1, t0 + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int d = 0;
  for (; d + 4 <= nd; d += 4) {
    dstage(d, 0, true);
    dstage(d + 1, 1, false);
    dstage(d + 2, 0, false);
    dstage(d + 3, 1, false);
  }
  if (d < nd) dstage(d, 0, false);
  if (d + 1 < nd) dstage(d + 1, 1, false);
  if (d + 2 < nd) dstage(d + 2, 0, false);

  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  uint16_t* blk = (uint16_t*)&sm.x[0][0] + wave * 32 * kStoreRowPad(FN);
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  const int64_t n_base = (int64_t)n0 + wave_n * FN * 32;
  store_tile_lds<FM, FN, kRowwise>(acc, p, Alpha{p.alpha, 0}, (int64_t)m0 + xg0 * 32, n_base,
                                   lane, blk);
  store_tile_lds<1, kS, kRowwise>(*(const floatx16(*)[kS][1])&accs, p, Alpha{p.alpha, 0},
                                  (int64_t)m0 + GS * 32, n_base + kI0 * 32, lane, blk);
}

template <int BM, int BN, bool kRowwise, int kFw, int kFx>
__global__ void __launch_bounds__(256) gemm_mx_fit_kernel(GemmProblem p) {
  __shared__ MxFitSmem<BM, BN> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  int tile_m, tile_n;
  tile_order(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  constexpr int FN = BN / 64;
  if ((wave >> 1) == 0)
    mx_fit_wave<BM, BN, kRowwise, FN - 1, kFw, kFx>(p, sm, lane, wave, tile_m * BM, tile_n * BN);
  else
    mx_fit_wave<BM, BN, kRowwise, 1, kFw, kFx>(p, sm, lane, wave, tile_m * BM, tile_n * BN);
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

// The same for the bf8 conversion against the software E5M2 encoder (clamp to
// [-57344, 57344], nearest, ties to even, saturating at 57344).
__global__ void mx_selftest_e5m2_exhaustive_kernel(unsigned long long* __restrict__ count,
                                                   uint32_t* __restrict__ first) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t nthreads = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u = tid; u < (1ull << 32); u += nthreads) {
    const uint32_t bits = (uint32_t)u;
    if (((bits >> 23) & 0xFFu) == 0xFFu) continue;
    const float y = __builtin_fminf(__builtin_fmaxf(u2f(bits), -kE5M2Max), kE5M2Max);
    const uint32_t hw = __builtin_amdgcn_cvt_pk_bf8_f32(y, 0.0f, 0, false) & 0xFFu;
    const uint32_t sw = ((bits >> 31) << 7) | e5m2_encode_sat(__builtin_fabsf(y));
    if (hw != sw) {
      const unsigned long long k = atomicAdd(count, 1ull);
      if (k < 16) first[k] = bits;
    }
  }
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int64_t M, int64_t K, void* codes, void* scales,
                              hipStream_t stream, const LaunchInfo& dev, MxElement elem) {
  const int64_t nlanes = M * K / 8;
  if (nlanes == 0) return hipSuccess;
  constexpr int kThreads = 256, kUnroll = 2;
  const int64_t want = (nlanes + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  const int64_t cap = (int64_t)dev.num_cus * 32;
  const int grid = (int)(want < cap ? want : cap);
  if (elem == MxElement::kE5M2)
    hipLaunchKernelGGL((mx_quantize_kernel<kUnroll, true>), dim3(grid), dim3(kThreads), 0, stream,
                       (const u32x4*)x, (u32x2*)codes, (uint8_t*)scales, nlanes);
  else
    hipLaunchKernelGGL((mx_quantize_kernel<kUnroll, false>), dim3(grid), dim3(kThreads), 0, stream,
                       (const u32x4*)x, (u32x2*)codes, (uint8_t*)scales, nlanes);
  return hipGetLastError();
}

namespace {

// 288 x 192 or 256 x 256 tiles: the fit tile issues 14 MFMAs per wave and stage (the
// other 16), so it wins unless it needs more passes over the compute units.
template <bool kRowwise, int kFw, int kFx>
hipError_t launch_fp8_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev) {
  const int64_t cus = dev.num_cus > 0 ? dev.num_cus : 256;
  const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  const int64_t tfit = ((p.M + 287) / 288) * ((p.N + 191) / 192);
  const bool fit32 = fits_i31(p.M + 320, p.K) && fits_i31(p.N + 192, p.K);
  const int64_t pass256 = (t256 + cus - 1) / cus, passfit = (tfit + cus - 1) / cus;
  if (fit32 && passfit * 14 <= pass256 * 16) {
    if (tfit > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_mx_fit_kernel<288, 192, kRowwise, kFw, kFx>), dim3((unsigned)tfit), dim3(256), 0,
                       stream, p);
  } else {
    if (t256 > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_mx_kernel<256, 256, kRowwise, kFw, kFx>), dim3((unsigned)t256), dim3(256), 0,
                       stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev,
                          MxElement a_elem, MxElement w_elem) {
  const bool a5 = a_elem == MxElement::kE5M2, w5 = w_elem == MxElement::kE5M2;
  if (w5 && a5) return launch_fp8_gemm<false, 1, 1>(p, stream, dev);
  if (w5) return launch_fp8_gemm<false, 1, 0>(p, stream, dev);
  if (a5) return launch_fp8_gemm<false, 0, 1>(p, stream, dev);
  return launch_fp8_gemm<false, 0, 0>(p, stream, dev);
}

hipError_t launch_fp8r_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev) {
  return launch_fp8_gemm<true, 0, 0>(p, stream, dev);
}

hipError_t launch_mx_selftest_e4m3_exhaustive(unsigned long long* count, uint32_t* first,
                                              hipStream_t stream) {
  hipLaunchKernelGGL(mx_selftest_e4m3_exhaustive_kernel, dim3(8192), dim3(256), 0, stream, count,
                     first);
  return hipGetLastError();
}

hipError_t launch_mx_selftest_e5m2_exhaustive(unsigned long long* count, uint32_t* first,
                                              hipStream_t stream) {
  hipLaunchKernelGGL(mx_selftest_e5m2_exhaustive_kernel, dim3(8192), dim3(256), 0, stream, count,
                     first);
  return hipGetLastError();
}

}  // namespace nvfp4
