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
//  * Packed 4-bit tiles and scale bytes stream from HBM into LDS (the direct-to-LDS
//    kernels load two stages of K, 256 elements or one 128-byte line of codes per row, at
//    a time into double-stage buffers; the register-staged kernel has two stage buffers);
//    decode happens in registers right before the MFMA, so LDS holds 4-bit data and its
//    traffic stays 4x below an f16-staged design.
//  * LDS layout of a packed tile: a lane reads its operand fragment for a 64-element
//    chunk (row r, bytes [16h, 16h+16) of the chunk) with one 16-byte LDS load, free of
//    bank conflicts. The direct-to-LDS kernels (288 x 192, 256 x 256, 128 x 192,
//    128 x 128, 128 x 64, and the 64 x 64 tile whose waves split K) keep each row's 128
//    bytes of a double stage together in 1 KiB pieces of 8 rows (16-byte chunks swizzled
//    by x_swz), because their loads read whole 128-byte lines; the register-staged kernel
//    stores 64 slots of 16 bytes per 32-row group and chunk in MFMA lane order.
//  * K mapping: lane half h of a fragment feeds the MFMA's K slots [8h, 8h+8) with
//    elements 32h + 8j .. 32h + 8j + 7 of the chunk on k-step j (j = 0..3). Both
//    operands use the same mapping, so each product pairs equal k; each lane's 8
//    elements sit inside one 16-element block and share one scale.
//  * Decode: the gfx950 conversion v_cvt_scalef32_pk_f16_fp4 turns two codes into two
//    f16 values, v_cvt_scalef32_pk_f16_fp8 turns a lane's two E4M3 scale bytes into f16,
//    and one packed f16 multiply per pair gives q * s exactly (all values are normal
//    f16, so no step depends on the denormal mode).
//  * The weights are the MFMA's A operand and the activations its B operand, so each
//    lane ends up holding 4 consecutive output columns of one row.
//  * Epilogue: fp32 accumulator * a_global * w_global (one fp32 multiply; split_alpha
//    adds an exact power-of-two ldexp for scale pairs whose product leaves the normal
//    binary32 range), round to nearest even bf16. The tiled direct-to-LDS kernels pass
//    each 32-row group of a wave's blocks through LDS and store 16-byte row pieces; the
//    others (and the 64 x 64 tile, after adding its partial tiles) store each lane's 8
//    bytes directly.
//  * Short activations (split-K kernel): K is split over the waves of a workgroup and
//    the partial sums meet in LDS; nvfp4_linear's fused form quantizes the activations
//    into LDS first. A few hundred rows: 64 x 64 tiles whose four waves each compute the
//    whole tile over a quarter of K, their partial tiles added in LDS.
#include "gemm_common.hpp"
#include "quant_common.hpp"

// VALU instructions the scheduler is asked to place after each MFMA of a k-step.
#ifndef NVFP4_GEMM_VALU_PER_MFMA
#define NVFP4_GEMM_VALU_PER_MFMA 5
#endif

namespace nvfp4 {

namespace {

template <int BM, int BN, int KC>
struct alignas(16) GemmSmem {
  uint8_t x[2][KC][BM * 32];   // activations, fragment order
  uint8_t w[2][KC][BN * 32];   // weights, fragment order
  uint32_t xs[2][KC][BM];      // 4 activation scale bytes per row and chunk
  uint32_t ws[2][KC][BN];      // 4 weight scale bytes per row and chunk
};

// Registers that carry one stage from global memory to LDS.
template <int ROWS, int KC, int NT>
struct StageRegs {
  static_assert((ROWS * KC * 2) % NT == 0, "pieces must divide evenly among threads");
  static constexpr int kPieces = ROWS * KC * 2 / NT;  // 16-byte pieces per thread
  static constexpr int kScales = (ROWS * KC + NT - 1) / NT;
  static constexpr bool kScalesExact = (ROWS * KC) % NT == 0;
  u32x4 piece[kPieces];
  uint32_t scale[kScales];
};

// Load one operand's stage: ROWS rows from row0, K chunks [k64, k64 + KC) of 64 elements.
// Consecutive threads take consecutive 16-byte pieces of the same row (a row holds
// 2*KC pieces per stage), so a wave reads whole cache lines. Rows past nrows repeat the
// last row (their results are never stored). kFast: K is a multiple of 64*KC and the
// operands are 16-byte (packed) / 4-byte (scales) aligned; otherwise pieces and scale
// bytes past K read as zero (a zero scale makes the decoded value zero).
template <int ROWS, int KC, int NT, bool kFast>
__device__ __forceinline__ void load_stage(StageRegs<ROWS, KC, NT>& r, const uint8_t* __restrict__ packed,
                                           const uint8_t* __restrict__ scales, int64_t row0,
                                           int64_t nrows, int64_t K, int64_t k64, int tid) {
  const int64_t pitch = K >> 1;
  const int64_t spitch = K >> 4;
#pragma unroll
  for (int p = 0; p < StageRegs<ROWS, KC, NT>::kPieces; ++p) {
    const int i = tid + p * NT;
    const int row = i / (2 * KC);
    const int q = i % (2 * KC);  // chunk * 2 + half
    int64_t grow = row0 + row;
    grow = grow < nrows ? grow : nrows - 1;
    const int64_t kel = (k64 + (q >> 1)) * 64 + (q & 1) * 32;  // first element of the piece
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
  for (int q = 0; q < StageRegs<ROWS, KC, NT>::kScales; ++q) {
    const int i = tid + q * NT;
    if (StageRegs<ROWS, KC, NT>::kScalesExact || i < ROWS * KC) {
      const int row = i / KC;
      const int kc = i % KC;
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

// Store a stage into LDS in MFMA fragment order (see the file comment).
template <int ROWS, int KC, int NT>
__device__ __forceinline__ void store_stage(const StageRegs<ROWS, KC, NT>& r, uint8_t (*dst)[ROWS * 32],
                                            uint32_t (*dscale)[ROWS], int tid) {
#pragma unroll
  for (int p = 0; p < StageRegs<ROWS, KC, NT>::kPieces; ++p) {
    const int i = tid + p * NT;
    const int row = i / (2 * KC);
    const int q = i % (2 * KC);
    const int slot = (row >> 5) * 64 + (q & 1) * 32 + (row & 31);
    *(u32x4*)&dst[q >> 1][slot * 16] = r.piece[p];
  }
#pragma unroll
  for (int q = 0; q < StageRegs<ROWS, KC, NT>::kScales; ++q) {
    const int i = tid + q * NT;
    if (StageRegs<ROWS, KC, NT>::kScalesExact || i < ROWS * KC) dscale[i % KC][i / KC] = r.scale[q];
  }
}

// WM x WN waves; wave (wave_m, wave_n) owns activation rows [wave_m*WTM, +WTM) and
// weight rows (output columns) [wave_n*WTN, +WTN) of the BM x BN tile.
template <int BM, int BN, int KC, int WM, int WN, bool kHw, bool kFast, bool kExp>
__global__ void __launch_bounds__(64 * WM * WN) gemm_kernel(GemmProblem p) {
  constexpr int NT = 64 * WM * WN;
  __shared__ GemmSmem<BM, BN, KC> sm;
  constexpr int WTM = BM / WM;  // activation rows per wave
  constexpr int WTN = BN / WN;  // weight rows (output columns) per wave
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tiles are multiples of 32");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_n = wave % WN;
  const int wave_m = wave / WN;

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

  StageRegs<BM, KC, NT> xr;
  StageRegs<BN, KC, NT> wr;
  load_stage<BM, KC, NT, kFast>(xr, p.a_packed, p.a_scales, m0, p.M, p.K, 0, tid);
  load_stage<BN, KC, NT, kFast>(wr, p.w_packed, p.w_scales, n0, p.N, p.K, 0, tid);
  store_stage<BM, KC, NT>(xr, sm.x[0], sm.xs[0], tid);
  store_stage<BN, KC, NT>(wr, sm.w[0], sm.ws[0], tid);
  __syncthreads();

  const int h = lane >> 5;
  const int r32 = lane & 31;

  // Main loop over K stages of KC chunks (64 elements each). The body is branch-free
  // (the prefetch issued on the last stage re-reads that stage) so the scheduler sees
  // one region per stage. Within a stage the k-steps (4 per chunk) are flattened: the
  // fragments of chunk c+1 are read from LDS while chunk c computes, and the decode of
  // k-step s+1 is issued before the MFMAs of k-step s, so VALU decode can overlap the
  // matrix core.
  constexpr int kSteps = 4 * KC;
  for (int64_t t = 0; t < nk; ++t) {
    const int buf = (int)(t & 1);
    const int64_t tn = t + 1 < nk ? t + 1 : t;
    load_stage<BM, KC, NT, kFast>(xr, p.a_packed, p.a_scales, m0, p.M, p.K, tn * KC, tid);
    load_stage<BN, KC, NT, kFast>(wr, p.w_packed, p.w_scales, n0, p.N, p.K, tn * KC, tid);
    // Keep the prefetch at the top of the stage: left to itself the scheduler sinks
    // these loads next to their LDS stores at the end of the body, exposing the whole
    // memory latency once per stage.
    __builtin_amdgcn_sched_barrier(0);

    u32x4 wraw[KC][FN], xraw[KC][FM];
    uint32_t wsr[KC][FN], xsr[KC][FM];  // the two scale bytes (blocks 2h, 2h+1) per fragment
    auto read_chunk = [&](int kc) {
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        wraw[kc][i] = *(const u32x4*)&sm.w[buf][kc][((wave_n * FN + i) * 64 + lane) * 16];
        wsr[kc][i] = *(const uint16_t*)((const uint8_t*)&sm.ws[buf][kc][wave_n * WTN + i * 32 + r32] + 2 * h);
      }
#pragma unroll
      for (int g = 0; g < FM; ++g) {
        xraw[kc][g] = *(const u32x4*)&sm.x[buf][kc][((wave_m * FM + g) * 64 + lane) * 16];
        xsr[kc][g] = *(const uint16_t*)((const uint8_t*)&sm.xs[buf][kc][wave_m * WTM + g * 32 + r32] + 2 * h);
      }
    };
    half2_t wsc[FN], xsc[FM];  // f16 scales of the chunk being decoded
    half8_t wf[2][FN], xf[2][FM];
    auto decode_step = [&](int st, half8_t* wo, half8_t* xo) {
      const int kc = st >> 2, j = st & 3;
      if (j == 0) {
#pragma unroll
        for (int i = 0; i < FN; ++i) wsc[i] = scales_to_f16<kHw>(wsr[kc][i]);
#pragma unroll
        for (int g = 0; g < FM; ++g) xsc[g] = scales_to_f16<kHw>(xsr[kc][g]);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) wo[i] = decode8<kHw>(wraw[kc][i][j], j < 2 ? wsc[i].xx : wsc[i].yy);
#pragma unroll
      for (int g = 0; g < FM; ++g) xo[g] = decode8<kHw>(xraw[kc][g][j], j < 2 ? xsc[g].xx : xsc[g].yy);
    };
    read_chunk(0);
    decode_step(0, wf[0], xf[0]);
    __builtin_amdgcn_sched_barrier(0);
    // One scheduling region per k-step: the MFMAs of step st, the decode of step st+1,
    // the LDS reads of the next chunk (on the first step of a chunk) and, on the last
    // step, the LDS stores of the prefetched stage. The group barriers ask for each MFMA
    // to be followed by a few VALU (and memory) instructions, so the decode runs in the
    // matrix core's shadow.
    constexpr int kMfmaPerStep = FN * FM;
    constexpr int kReadsPerChunk = 2 * (FN + FM);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int cur = st & 1;
      const bool reads = (st & 3) == 0 && (st >> 2) + 1 < KC;
      if (reads) read_chunk((st >> 2) + 1);
      if (st + 1 < kSteps) decode_step(st + 1, wf[cur ^ 1], xf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
      if (st + 1 == kSteps) {
        store_stage<BM, KC, NT>(xr, sm.x[buf ^ 1], sm.xs[buf ^ 1], tid);
        store_stage<BN, KC, NT>(wr, sm.w[buf ^ 1], sm.ws[buf ^ 1], tid);
      }
#pragma unroll
      for (int q = 0; q < kMfmaPerStep; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (reads && q < kReadsPerChunk) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        if (st + 1 == kSteps) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_GEMM_VALU_PER_MFMA, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  store_tile<FM, FN, kExp>(acc, p, gemm_alpha(p), m0 + wave_m * WTM, n0 + wave_n * WTN, lane);
}

// ---- 256 x 256, 128 x 192, 128 x 128 and 128 x 64 tiles: direct-to-LDS loads ----------
//
// 2 x 2 waves of BM/2 x BN/2: 4 x 4 blocks of 32 x 32 for 256 x 256 (the large-M tile),
// 2 x 3 for 128 x 192, 2 x 2 for 128 x 128 and 2 x 1 for 128 x 64 (medium M: more tiles,
// so fewer rows still fill the chip, at a higher decode cost per MFMA). Loads, LDS image
// and pipeline are the 288 x 192 kernel's (below): codes two stages at a time in 8-row x
// 128-byte pieces (x_swz chunk swizzle), a double stage's scales in 64-row x 16-byte
// pieces, two double-stage code buffers and two scale buffers, one wait and barrier per
// double stage inside its second stage; range-checked buffer loads over row windows
// (window_rsrc), so a ragged tile needs no clamping. 2 x 64 KiB + 2 x 8 KiB = 144 KiB of
// LDS at 256 x 256, 2 x 40 KiB + 2 x 5 KiB = 90 KiB at 128 x 192.
template <int BM, int BN>
struct alignas(16) GemmSmem256 {
  uint8_t x[2][BM * 128];
  uint8_t w[2][BN * 128];
  uint8_t sc[2][(BM + BN) * 16];
};

// Requires K % 128 == 0, 16-byte aligned packed operands, 4-byte aligned scales, and
// (rows + one tile) x K/2 below 2^31 for both operands (32-bit buffer offsets).
template <int BM, int BN, bool kExp>
__global__ void __launch_bounds__(256) gemm_dma_kernel(GemmProblem p) {
  constexpr int NW = 4, WM = 2, WN = 2;
  __shared__ GemmSmem256<BM, BN> sm;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int kSteps = 8;  // 16-element k-steps per stage (two chunks of 4)
  constexpr int kPx = BM / 8, kPw = BN / 8;  // 1 KiB code pieces per double stage
  static_assert((kPx + kPw) % NW == 0, "code pieces divide among waves");
  constexpr int kCode = (kPx + kPw) / NW;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole 64-row scale pieces");
  constexpr int kSp = (BM + BN) / 64;             // scale pieces per double stage
  constexpr int kScale = (kSp + NW - 1) / NW;     // per wave (the last piece repeated)
  constexpr int kLoads = kCode + kScale;
  static_assert(kLoads < 64, "a double stage of loads fits the vmcnt counter");
  constexpr int kLoadsPerStep = (kLoads + 3) / 4;  // over the odd stage's last 4 k-steps

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
  const int nk = (int)(p.K / 128);  // stages
  const int nd = (nk + 1) >> 1;     // double stages
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);

  // row windows [m0, M) and [n0, N) (see window_rsrc)
  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, m0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, m0, p.M, spitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);

  // load j of this wave for double stage ds into buffer buf: code pieces (activation
  // rows 8i .. 8i+7, then weight rows), then scale pieces (64 rows x 16 bytes, activation
  // rows first; slots past the last piece repeat it, writing the same bytes to the same
  // place)
  auto issue = [&](int j, int ds, int buf) {
    if (j < kCode) {
      const int i = j * NW + wave;
      const bool isx = i < kPx;
      const int prow = 8 * (isx ? i : i - kPx);
      buffer_load_lds16(isx ? rxp : rwp, isx ? &sm.x[buf][i * 1024] : &sm.w[buf][(i - kPx) * 1024],
                        x_piece_voff(lane, prow, pitch) + (uint32_t)ds * 128, 0);
    } else {
      const int i = min((j - kCode) * NW + wave, kSp - 1);
      const bool isx = i < BM / 64;
      const int prow = isx ? 64 * i : 64 * (i - BM / 64);
      buffer_load_lds16(isx ? rxs : rws, &sm.sc[buf][i * 1024],
                        scale_piece_voff(lane, prow, spitch, (uint32_t)ds * 16), 0);
    }
  };

  floatx16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  // fragments of two chunks and decoded operands of two k-steps
  const int rbase = (r32 >> 3) * 1024 + (r32 & 7) * 128;  // lane's row in a 32-row group
  const int sw = x_swz(r32);
  const int wfrag = wave_n * FN * 4096;
  const int xfrag = wave_m * FM * 4096;
  const int wsw = (BM + wave_n * WTN + r32) * 16 + 2 * h;
  const int xsw = (wave_m * WTM + r32) * 16 + 2 * h;
  u32x4 wraw[2][FN], xraw[2][FM];
  uint32_t wsr[2][FN], xsr[2][FM];
  half2_t wsc[FN], xsc[FM];
  half8_t wf[2][FN], xf[2][FM];
  // chunk c of stage half hs of the double stage in buffer buf, as chunk par
  auto read_chunk = [&](int par, int buf, int hs, int c) {
    const int fr = rbase + 16 * ((2 * (2 * hs + c) + h) ^ sw);
    const uint8_t* wb = &sm.w[buf][wfrag + fr];
    const uint8_t* xb = &sm.x[buf][xfrag + fr];
    const uint8_t* scb = &sm.sc[buf][hs * 8 + c * 4];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[par][i] = *(const u32x4*)(wb + i * 4096);
      wsr[par][i] = *(const uint16_t*)(scb + wsw + i * 512);
    }
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      xraw[par][g] = *(const u32x4*)(xb + g * 4096);
      xsr[par][g] = *(const uint16_t*)(scb + xsw + g * 512);
    }
  };
  auto decode_step = [&](int par, int j, half8_t* wo, half8_t* xo) {
    if (j == 0) {
#pragma unroll
      for (int i = 0; i < FN; ++i) wsc[i] = scales_to_f16<true>(wsr[par][i]);
#pragma unroll
      for (int g = 0; g < FM; ++g) xsc[g] = scales_to_f16<true>(xsr[par][g]);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) wo[i] = decode8<true>(wraw[par][i][j], j < 2 ? wsc[i].xx : wsc[i].yy);
#pragma unroll
    for (int g = 0; g < FM; ++g) xo[g] = decode8<true>(xraw[par][g][j], j < 2 ? xsc[g].xx : xsc[g].yy);
  };

  // prologue: double stages 0 and 1 (a double stage past the last reloads the last into
  // the free buffer); wait for 0 (1 may stay in flight), read its first chunk
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, nd > 1 ? 1 : 0, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 15) | ((kLoads >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  read_chunk(0, 0, 0, 0);
  decode_step(0, 0, wf[0], xf[0]);

  constexpr int kMfmaPerStep = FN * FM;
  constexpr int kReadsPerChunk = 2 * (FN + FM);
  // stage half hs (a constant) of double stage d in buffer b (a constant)
  auto stage = [&](int d, const int b, const int hs) {
    const int lds_ = d + 2 < nd ? d + 2 : nd - 1;  // double stage loaded into b at the end
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int cur = st & 1;
      const int j = st & 3;
      if (st == 0) read_chunk(1, b, hs, 1);  // this stage's second chunk
      if (st == 4) {
        if (hs == 0) {
          read_chunk(0, b, 1, 0);  // stage 2d+1's first chunk, same buffer
        } else {
          // vmcnt(0) and lgkmcnt(0): double stage d+1 loaded, this wave's reads of b done
          __builtin_amdgcn_s_waitcnt(0x0070);
          __builtin_amdgcn_s_barrier();
          read_chunk(0, b ^ 1, 0, 0);  // double stage d+1's first chunk
        }
      }
      const bool loads = hs == 1 && st >= 4;
      if (loads) {
#pragma unroll
        for (int l = 0; l < kLoadsPerStep; ++l)
          if ((st - 4) * kLoadsPerStep + l < kLoads) issue((st - 4) * kLoadsPerStep + l, lds_, b);
      }
      // decode of the next k-step (the first k-step of the next stage after the last)
      decode_step(((st + 1) >> 2) & 1, (st + 1) & 3, wf[cur ^ 1], xf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < kMfmaPerStep; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (j == 0 && q < kReadsPerChunk) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        if (loads && q < kLoadsPerStep && (st - 4) * kLoadsPerStep + q < kLoads)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS
        __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_GEMM_VALU_PER_MFMA, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int d = 0;
  for (; 2 * d + 4 <= nk; d += 2) {
    stage(d, 0, 0);
    stage(d, 0, 1);
    stage(d + 1, 1, 0);
    stage(d + 1, 1, 1);
  }
  if (2 * d < nk) stage(d, 0, 0);
  if (2 * d + 1 < nk) stage(d, 0, 1);
  if (2 * d + 2 < nk) stage(d + 1, 1, 0);

  // drain the last (unused) loads before the code buffers stage the stores
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  store_tile_lds<FM, FN, false, kExp>(acc, p, gemm_alpha(p), (int64_t)m0 + wave_m * WTM,
                                      (int64_t)n0 + wave_n * WTN, lane,
                                      (uint16_t*)&sm.x[0][0] + wave * 32 * kStoreRowPad(FN));
}

// ---- activations of a few hundred rows: the waves of a workgroup split K ----------------
//
// A few hundred activation rows fill the chip only with small tiles (64 or 128 rows);
// shared 2 x 2 among the waves those give each wave one or two blocks per operand, 1 to 1.5
// decoded fragments per MFMA, and the decode instead of the matrix pipe sets the pace.
// Here the waves split K as well as the tile: KS waves share each of the 4 / KS row bands
// of the BM x BN tile (a wave computes its whole band, RM x BN, on every KS-th stage), so
// a wave keeps more blocks per decoded fragment on a tile as small as before: 64 x 64 with
// KS = 4 (2 x 2 blocks per wave, one fragment per MFMA), 128 x 128 with KS = 2 (2 x 4
// blocks, 0.75). A set is KS stages (KS / 2 double stages) and wave w takes stage
// KS t + w % KS of set t. Loads and LDS image are the 256 x 256 kernel's (8-row x 128-byte
// code pieces and 64-row x 16-byte scale pieces per double stage); a set fills a group
// of double-stage buffers and two groups alternate. In each set a wave reads its stage's
// second chunk at once; at the fifth k-step it waits for the next set's loads (its LDS
// reads of this set are done by then), meets the workgroup at a barrier, reads the next
// set's first chunk and issues the loads of the set after that into the group every wave
// has finished reading. At the end the KS partial sums of every block meet in LDS (the
// pipeline's buffers, grown to hold all of them at once where needed) and are added in
// wave order (the same sums on every run).
template <int BM, int BN, int KS>
union alignas(16) GemmSmemWsplit {
  struct {
    uint8_t x[KS][BM * 128];
    uint8_t w[KS][BN * 128];
    uint8_t sc[KS][(BM + BN) * 16];
  } pipe;
  // the four waves' partial blocks (32 x 32 fp32 each) at the end
  float red[4][(BM / (4 / KS) / 32) * (BN / 32)][64 * 16];
};

// Requires K % (128 KS) == 0 (whole sets), 16-byte aligned packed operands, 4-byte
// aligned scales, and (rows + one tile) x K/2 below 2^31 for both operands.
template <int BM, int BN, int KS, bool kExp>
__global__ void __launch_bounds__(256) gemm_wsplit_kernel(GemmProblem p) {
  constexpr int NW = 4;
  static_assert(KS == 2 || KS == 4, "two or four waves per row band");
  constexpr int WM = NW / KS;         // row bands
  constexpr int RM = BM / WM;         // rows per band
  constexpr int FM = RM / 32, FN = BN / 32;
  constexpr int DS = KS / 2;          // double stages per set
  constexpr int kSteps = 8;  // 16-element k-steps per stage (two chunks of 4)
  constexpr int kPx = BM / 8, kPw = BN / 8;  // 1 KiB code pieces per double stage
  static_assert(RM % 32 == 0 && (kPx + kPw) % NW == 0, "whole blocks; code pieces divide among waves");
  constexpr int kCode = (kPx + kPw) / NW;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole 64-row scale pieces");
  constexpr int kSp = (BM + BN) / 64;          // scale pieces per double stage
  constexpr int kScale = (kSp + NW - 1) / NW;  // per wave (the last piece repeated)
  constexpr int kLoadsDs = kCode + kScale;     // per wave and double stage
  constexpr int kLoads = DS * kLoadsDs;        // per wave and set
  static_assert(kLoads < 64, "a set of loads fits the vmcnt counter");
  constexpr int kLoadsPerStep = (kLoads + 3) / 4;  // over a set's last 4 k-steps
  constexpr int kMfmaPerStep = FN * FM;
  constexpr int kReadsPerChunk = 2 * (FN + FM);
  constexpr int kReadsPerMfma = (kReadsPerChunk + kMfmaPerStep - 1) / kMfmaPerStep;
  constexpr int kValuPerMfma = (8 * (FN + FM) + kMfmaPerStep - 1) / kMfmaPerStep;
  __shared__ GemmSmemWsplit<BM, BN, KS> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const int wm = wave / KS;   // the wave's row band
  const int wk = wave % KS;   // and stage within a set
  const int wq = wk >> 1;     // its double stage within the set
  const int whs = wk & 1;     // and stage within that

  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  int tile_m, tile_n;
  tile_order(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;
  const int nset = (int)(p.K / (128 * KS));
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);

  // row windows [m0, M) and [n0, N) (see window_rsrc)
  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, m0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, m0, p.M, spitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);

  // load j (0 .. kLoads - 1) of this wave for set t into buffer group grp: per double
  // stage DS t + j / kLoadsDs, code pieces (activation rows 8i .. 8i+7, then weight rows),
  // then scale pieces (64 rows x 16 bytes, activation rows first; slots past the last
  // piece repeat it, writing the same bytes to the same place)
  auto issue = [&](int j, int t, int grp) {
    const int half = j / kLoadsDs;
    const int jj = j - half * kLoadsDs;
    const int ds = DS * t + half;
    const int buf = DS * grp + half;
    if (jj < kCode) {
      const int i = jj * NW + wave;
      const bool isx = i < kPx;
      const int prow = 8 * (isx ? i : i - kPx);
      buffer_load_lds16(isx ? rxp : rwp, isx ? &sm.pipe.x[buf][i * 1024] : &sm.pipe.w[buf][(i - kPx) * 1024],
                        x_piece_voff(lane, prow, pitch) + (uint32_t)ds * 128, 0);
    } else {
      const int i = min((jj - kCode) * NW + wave, kSp - 1);
      const bool isx = i < BM / 64;
      const int prow = isx ? 64 * i : 64 * (i - BM / 64);
      buffer_load_lds16(isx ? rxs : rws, &sm.pipe.sc[buf][i * 1024],
                        scale_piece_voff(lane, prow, spitch, (uint32_t)ds * 16), 0);
    }
  };

  floatx16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  // fragments of two chunks and decoded operands of two k-steps
  const int rbase = (r32 >> 3) * 1024 + (r32 & 7) * 128;  // lane's row in a 32-row group
  const int sw = x_swz(r32);
  const int xfrag = wm * FM * 4096;
  const int wsw = (BM + r32) * 16 + 2 * h;
  const int xsw = (wm * RM + r32) * 16 + 2 * h;
  u32x4 wraw[2][FN], xraw[2][FM];
  uint32_t wsr[2][FN], xsr[2][FM];
  half2_t wsc[FN], xsc[FM];
  half8_t wf[2][FN], xf[2][FM];
  // chunk c of this wave's stage of the set in buffer group grp, as chunk par
  auto read_chunk = [&](int par, int grp, int c) {
    const int buf = DS * grp + wq;
    const int fr = rbase + 16 * ((2 * (2 * whs + c) + h) ^ sw);
    const uint8_t* wb = &sm.pipe.w[buf][fr];
    const uint8_t* xb = &sm.pipe.x[buf][xfrag + fr];
    const uint8_t* scb = &sm.pipe.sc[buf][whs * 8 + c * 4];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[par][i] = *(const u32x4*)(wb + i * 4096);
      wsr[par][i] = *(const uint16_t*)(scb + wsw + i * 512);
    }
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      xraw[par][g] = *(const u32x4*)(xb + g * 4096);
      xsr[par][g] = *(const uint16_t*)(scb + xsw + g * 512);
    }
  };
  auto decode_step = [&](int par, int j, half8_t* wo, half8_t* xo) {
    if (j == 0) {
#pragma unroll
      for (int i = 0; i < FN; ++i) wsc[i] = scales_to_f16<true>(wsr[par][i]);
#pragma unroll
      for (int g = 0; g < FM; ++g) xsc[g] = scales_to_f16<true>(xsr[par][g]);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) wo[i] = decode8<true>(wraw[par][i][j], j < 2 ? wsc[i].xx : wsc[i].yy);
#pragma unroll
    for (int g = 0; g < FM; ++g) xo[g] = decode8<true>(xraw[par][g][j], j < 2 ? xsc[g].xx : xsc[g].yy);
  };

  // prologue: sets 0 and 1 into groups 0 and 1; wait for set 0, read its first chunk
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, 0, 0);
  if (nset > 1) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) issue(j, 1, 1);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 15) | ((kLoads >> 4) << 14));
  } else {
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  read_chunk(0, 0, 0);
  decode_step(0, 0, wf[0], xf[0]);

  // set t in buffer group grp (a constant); loads: issue set t + 2 into grp (a constant);
  // last: no set follows (a constant)
  auto set = [&](int t, const int grp, const bool loads, const bool last) {
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int cur = st & 1;
      const int j = st & 3;
      if (st == 0) read_chunk(1, grp, 1);  // this stage's second chunk
      if (st == 4 && !last) {
        // vmcnt(0) and lgkmcnt(0): set t + 1 loaded, this wave's reads of group grp done
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        read_chunk(0, grp ^ 1, 0);  // set t + 1's first chunk
      }
      const bool ld = loads && st >= 4;
      if (ld) {
#pragma unroll
        for (int l = 0; l < kLoadsPerStep; ++l)
          if ((st - 4) * kLoadsPerStep + l < kLoads) issue((st - 4) * kLoadsPerStep + l, t + 2, grp);
      }
      // decode of the next k-step (the first k-step of the next set after the last)
      if (!(last && st + 1 == kSteps)) decode_step(((st + 1) >> 2) & 1, (st + 1) & 3, wf[cur ^ 1], xf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < kMfmaPerStep; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (j == 0 && q * kReadsPerMfma < kReadsPerChunk)
          __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerMfma, 0);  // LDS reads
        if (ld && q < kLoadsPerStep && (st - 4) * kLoadsPerStep + q < kLoads)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // sets in pairs while two more follow, then the last one to three
  int t = 0;
  for (; t + 4 <= nset; t += 2) {
    set(t, 0, true, false);
    set(t + 1, 1, true, false);
  }
  const int rest = nset - t;
  if (rest == 3) {
    set(t, 0, true, false);
    set(t + 1, 1, false, false);
    set(t + 2, 0, false, true);
  } else if (rest == 2) {
    set(t, 0, false, false);
    set(t + 1, 1, false, true);
  } else {
    set(t, 0, false, true);
  }

  // The KS partial sums of every block meet in LDS (each wave writes all its blocks, four
  // values per lane and 16-byte access, consecutive lanes side by side); among the KS
  // waves of a row band, wave wk adds the parts of every KS-th block in wave order,
  // scales and stores it.
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  typedef float floatx4 __attribute__((ext_vector_type(4)));
  constexpr int NB = FN * FM;  // blocks per wave
  static_assert(sizeof(sm.red[0]) == NB * 64 * 16 * sizeof(float), "partial blocks");
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      *(floatx4*)&sm.red[wave][b][(v4 * 64 + lane) * 4] =
          floatx4{acc[b / FM][b % FM][4 * v4], acc[b / FM][b % FM][4 * v4 + 1],
                  acc[b / FM][b % FM][4 * v4 + 2], acc[b / FM][b % FM][4 * v4 + 3]};
  __syncthreads();
  const Alpha alpha = gemm_alpha(p);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b % KS != wk) continue;
    floatx16 tot[1][1];
#pragma unroll
    for (int src = 0; src < KS; ++src)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const floatx4 part = *(const floatx4*)&sm.red[wm * KS + src][b][(v4 * 64 + lane) * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tot[0][0][4 * v4 + e] = src == 0 ? part[e] : tot[0][0][4 * v4 + e] + part[e];
      }
    store_tile<1, 1, kExp>(tot, p, alpha, (int64_t)m0 + wm * RM + (b % FM) * 32,
                           (int64_t)n0 + (b / FM) * 32, lane);
  }
}

// ---- fit-tile path: 288 x 192 tiles ------------------------------------------------------
//
// The 256x256 tile leaves part of the chip idle at the token count of a 1024x1024 FLUX
// image: 4608 = 18 x 256 rows against 256 compute units gives 216 tiles for a 3072-wide
// output. 4608 = 16 x 288 and every FLUX width (3072, 9216, 12288) is a multiple of 192,
// so a 288 x 192 tile splits these products into whole multiples of 256 tiles.
//
// The tile is 9 x 6 blocks of 32 x 32 outputs (the 32x32x16 MFMA), which 4 waves cannot
// share evenly. Wave (m, n) owns weight groups 3n..3n+2 and activation groups 0..3 (m = 0)
// or 5..8 (m = 1) over the whole K range, plus the middle activation group 4 over one of
// the two 64-element chunks of every 128-element stage. Each wave runs "its" chunk first
// (wave m = 0 physical chunk 0, m = 1 chunk 1) and takes group 4 there, so all waves run
// one program: 13.5 blocks of work per wave and k-step on average. At the end the two
// partial sums of group 4 meet in LDS.
//
// Loads. The direct-to-LDS path costs by the cache lines an instruction touches rather
// than by its bytes (measured on the device: 88.6 GB/s per compute unit of L2-resident
// data for 8 rows x 128 bytes per load, 51.3 for 16 rows x 64 bytes), so the codes are
// loaded two stages (256 elements of K: a whole 128-byte line per row) at a time, 8 rows x
// 128 bytes per load, and a double stage's scales (16 bytes per row) 64 rows per load.
// LDS: two double-stage code buffers and two scale buffers (136 KiB); each row's 128
// bytes as eight 16-byte chunks at slots q ^ x_swz(row % 32), so the fragment reads (lane
// (h, r) of chunk c of the double stage reads 16-byte chunk 2c + h of row r) hit distinct
// banks. Scales: activation rows (rounded up to whole 64-row pieces) first, then weight
// rows. The double stage's byte offset along the row rides in the per-lane offset, so for
// an odd number of stages the unused second half of the last double stage is
// range-checked like any load (zero past the operand's end).
//
// Pipeline over double stages d (stages 2d, 2d+1, buffers d & 1), each stage's chunks in
// the wave's own order:
//  * stage 2d reads its second chunk and then stage 2d+1's first chunk from the same
//    buffer under its MFMAs;
//  * stage 2d+1 reads its second chunk under its first k-steps; then the wave waits for
//    all its loads (double stage d+1's, issued during stage 2d-1) with its LDS reads
//    landed and meets the workgroup at a barrier, reads double stage d+1's first chunk,
//    and issues double stage d+2's loads into buffer d & 1, whose reads all ended before
//    the barrier.
// Each k-step decodes the next one's fragments under its MFMAs.
template <int BM, int BN>
struct alignas(16) GemmSmemFit {
  static constexpr int kScaleRowsX = (BM + 63) / 64 * 64;
  uint8_t x[2][BM * 128];
  uint8_t w[2][BN * 128];
  uint8_t sc[2][(kScaleRowsX + BN) * 16];
};

// Requires K % 128 == 0, 16-byte aligned packed operands, 4-byte aligned scales, and
// (rows + one tile) x K/2 below 2^31 for both operands (32-bit buffer offsets).
template <int BM, int BN, bool kExp>
__global__ void __launch_bounds__(256) gemm_fit_kernel(GemmProblem p) {
  constexpr int NW = 4;
  constexpr int GX = BM / 32, GW = BN / 32;
  static_assert(GX * 32 == BM && GW * 32 == BN, "tiles are whole 32-row groups");
  static_assert(GX % 2 == 1 && GW % 2 == 0, "odd activation groups, even weight groups");
  constexpr int FM = GX / 2;  // whole activation groups per wave
  constexpr int FN = GW / 2;  // weight groups per wave
  constexpr int GS = FM;      // the shared middle activation group
  constexpr int kSteps = 8;   // 16-element k-steps per stage (two chunks of 4)
  __shared__ GemmSmemFit<BM, BN> sm;

  constexpr int kPx = BM / 8, kPw = BN / 8;  // 1 KiB code pieces per double stage
  static_assert((kPx + kPw) % NW == 0, "code pieces divide among waves");
  constexpr int kCode = (kPx + kPw) / NW;
  constexpr int kRowsSx = GemmSmemFit<BM, BN>::kScaleRowsX;
  constexpr int kSx = kRowsSx / 64;
  static_assert(BN % 64 == 0 && kSx + BN / 64 == 2 * NW, "two scale loads per wave and double stage");
  constexpr int kLoads = kCode + 2;                   // per wave and double stage
  static_assert(kLoads < 64, "a double stage of loads fits the vmcnt counter");
  constexpr int kLoadsPerStep = (kLoads + 3) / 4;     // over the odd stage's last 4 k-steps

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_n = wave & 1;
  const int wave_m = wave >> 1;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  int tile_m, tile_n;
  tile_order(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;
  const int nk = (int)(p.K / 128);      // stages
  const int nd = (nk + 1) >> 1;         // double stages (the last one half used when nk is odd)
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);

  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, m0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, m0, p.M, spitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);

  // Load j of this wave for double stage ds into buffer buf: code pieces (activation
  // rows 8i .. 8i+7, then weight rows), then the two scale pieces (64 rows x 16 bytes;
  // activation rows first, selects, no branch).
  auto issue = [&](int j, int ds, int buf) {
    if (j < kCode) {
      const int i = j * NW + wave;
      const bool isx = i < kPx;
      const int prow = 8 * (isx ? i : i - kPx);
      buffer_load_lds16(isx ? rxp : rwp, isx ? &sm.x[buf][i * 1024] : &sm.w[buf][(i - kPx) * 1024],
                        x_piece_voff(lane, prow, pitch) + (uint32_t)ds * 128, 0);
    } else {
      const int i = (j - kCode) * NW + wave;
      const bool isx = i < kSx;
      const int prow = isx ? 64 * i : 64 * (i - kSx);
      buffer_load_lds16(isx ? rxs : rws, &sm.sc[buf][i * 1024],
                        scale_piece_voff(lane, prow, spitch, (uint32_t)ds * 16), 0);
    }
  };

  floatx16 acc[FN][FM], accs[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) accs[i][v] = 0.0f;
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;
  }

  const int xg0 = wave_m ? GS + 1 : 0;  // first whole activation group of this wave
  const int rbase = (r32 >> 3) * 1024 + (r32 & 7) * 128;  // lane's row in a 32-row group
  const int sw = x_swz(r32);
  const int wfrag = wave_n * FN * 4096;
  const int xfrag = xg0 * 4096;
  const int sfrag = GS * 4096;
  const int wsw = (kRowsSx + wave_n * FN * 32 + r32) * 16 + 2 * h;  // scale byte offsets
  const int xsw = (xg0 * 32 + r32) * 16 + 2 * h;
  const int ssw = (GS * 32 + r32) * 16 + 2 * h;
  u32x4 wraw[2][FN], xraw[2][FM], sraw;
  uint32_t wsr[2][FN], xsr[2][FM], ssr;
  half2_t wsc[FN], xsc[FM], ssc;
  half8_t wf[2][FN], xf[2][FM], sf[2];
  // read chunk cc (physical, 0 or 1) of stage half hs of the double stage in buffer buf
  // as the wave's chunk par; the shared group only in its first chunk
  auto read_chunk = [&](int par, int buf, int hs, int cc) {
    const int fr = rbase + 16 * ((2 * (2 * hs + cc) + h) ^ sw);
    const uint8_t* wb = &sm.w[buf][wfrag + fr];
    const uint8_t* xb = &sm.x[buf][xfrag + fr];
    const uint8_t* scb = &sm.sc[buf][hs * 8 + cc * 4];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[par][i] = *(const u32x4*)(wb + i * 4096);
      wsr[par][i] = *(const uint16_t*)(scb + wsw + i * 512);
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      xraw[par][f] = *(const u32x4*)(xb + f * 4096);
      xsr[par][f] = *(const uint16_t*)(scb + xsw + f * 512);
    }
    if (par == 0) {
      sraw = *(const u32x4*)&sm.x[buf][sfrag + fr];
      ssr = *(const uint16_t*)(scb + ssw);
    }
  };
  auto decode_step = [&](int par, int j, int slot) {
    if (j == 0) {
#pragma unroll
      for (int i = 0; i < FN; ++i) wsc[i] = scales_to_f16<true>(wsr[par][i]);
#pragma unroll
      for (int f = 0; f < FM; ++f) xsc[f] = scales_to_f16<true>(xsr[par][f]);
      if (par == 0) ssc = scales_to_f16<true>(ssr);
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[slot][i] = decode8<true>(wraw[par][i][j], j < 2 ? wsc[i].xx : wsc[i].yy);
#pragma unroll
    for (int f = 0; f < FM; ++f) xf[slot][f] = decode8<true>(xraw[par][f][j], j < 2 ? xsc[f].xx : xsc[f].yy);
    if (par == 0) sf[slot] = decode8<true>(sraw[j], j < 2 ? ssc.xx : ssc.yy);
  };

  // prologue: double stages 0 and 1 (a double stage past the last reloads the last into
  // the free buffer); wait for 0 (1 may stay in flight), read its first chunk
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, nd > 1 ? 1 : 0, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 15) | ((kLoads >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  read_chunk(0, 0, 0, wave_m);
  decode_step(0, 0, 0);

  // stage half hs (a constant) of double stage d in buffer b (a constant)
  auto stage = [&](int d, const int b, const int hs) {
    const int lds_ = d + 2 < nd ? d + 2 : nd - 1;  // double stage loaded into b at the end
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int cur = st & 1;
      const int par = st >> 2, j = st & 3;
      if (st == 0) read_chunk(1, b, hs, wave_m ^ 1);  // this stage's second chunk
      if (st == 4) {
        if (hs == 0) {
          read_chunk(0, b, 1, wave_m);  // stage 2d+1's first chunk, same buffer
        } else {
          // vmcnt(0) and lgkmcnt(0): double stage d+1 loaded, this wave's reads of b done
          __builtin_amdgcn_s_waitcnt(0x0070);
          __builtin_amdgcn_s_barrier();
          read_chunk(0, b ^ 1, 0, wave_m);  // double stage d+1's first chunk
        }
      }
      const bool loads = hs == 1 && st >= 4;
      if (loads) {
#pragma unroll
        for (int l = 0; l < kLoadsPerStep; ++l)
          if ((st - 4) * kLoadsPerStep + l < kLoads) issue((st - 4) * kLoadsPerStep + l, lds_, b);
      }
      decode_step(((st + 1) >> 2) & 1, (st + 1) & 3, cur ^ 1);
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][i], xf[cur][f], acc[i][f], 0, 0, 0);
        if (par == 0) accs[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][i], sf[cur], accs[i], 0, 0, 0);
      }
      constexpr int kReads = 2 * (FN + FM) + 2;
      const int nmfma = FN * FM + (par == 0 ? FN : 0);
#pragma unroll
      for (int q = 0; q < FN * (FM + 1); ++q) {
        if (q < nmfma) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          if (j == 0 && q < kReads / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
          if (loads && q < kLoadsPerStep && (st - 4) * kLoadsPerStep + q < kLoads)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS
          __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_GEMM_VALU_PER_MFMA, 0);  // VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int d = 0;
  for (; 2 * d + 4 <= nk; d += 2) {
    stage(d, 0, 0);
    stage(d, 0, 1);
    stage(d + 1, 1, 0);
    stage(d + 1, 1, 1);
  }
  if (2 * d < nk) stage(d, 0, 0);
  if (2 * d + 1 < nk) stage(d, 0, 1);
  if (2 * d + 2 < nk) stage(d + 1, 1, 0);

  // The two partial sums of the shared group: drain the last (unused) loads, then swap
  // them through LDS (the buffers are free now).
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  float* xch = (float*)&sm.x[0][0];
  static_assert(NW * FN * 16 * 64 * sizeof(float) <= sizeof(sm.x), "exchange fits");
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) xch[((wave * FN + i) * 16 + v) * 64 + lane] = accs[i][v];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) accs[i][v] += xch[(((wave ^ 2) * FN + i) * 16 + v) * 64 + lane];

  const int64_t n_base = (int64_t)n0 + wave_n * FN * 32;
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.w), "store staging fits");
  const Alpha alpha = gemm_alpha(p);
  store_tile_lds<FM, FN, false, kExp>(acc, p, alpha, (int64_t)m0 + xg0 * 32, n_base, lane,
                                      (uint16_t*)&sm.w[0][0] + wave * 32 * kStoreRowPad(FN));
  // group GS: wave m = 0 stores column quads 0-1 of every block, m = 1 quads 2-3
  store_tile<1, FN, kExp>(*(const floatx16(*)[FN][1])&accs, p, alpha, (int64_t)m0 + GS * 32,
                          n_base, lane, wave_m * 2, wave_m * 2 + 2);
}

// Fused linear for the shortest activations: the workgroup quantizes the M x K bf16
// activations (M * K <= kFuseElems, or kFuseElemsGemv in the 16-row kernel) into LDS in the NVFP4 layout (codes xq [M][K/2], scales
// xqs [M][K/16]) with the quantize kernel's functions, so codes and scales are bit-identical
// to nvfp4_quantize's, and with `store` also into the caller's workspace. Half block hb
// (8 elements) per lane, the pair (hb, hb ^ 1) being one block in lanes (2i, 2i + 1) of one
// wave; the workgroup's `nthreads` threads (a multiple of 64) take half blocks in turn, U
// at a time (their loads issued first), so both lanes of a pair are always active
// together.
constexpr int kFuseElems = 16384;      // split-K's fused form
constexpr int kFuseElemsGemv = 24576;  // the 16-row kernel's fused form (12 KiB of codes)
__device__ __forceinline__ void quantize_to_lds(const FusedQuant& fq, int64_t M, int64_t K,
                                                uint8_t* xq, uint8_t* xqs, bool store,
                                                int nthreads) {
  constexpr int U = 4;  // loads in flight per thread before their half blocks are encoded
  const QuantScale qsc = quant_scale(fq.gs, fq.den, fq.rden, fq.gs_dev);
  const int nhalves = (int)(M * K / 8);
  const u32x4* xv = (const u32x4*)fq.x;
  for (int base = threadIdx.x; base < nhalves; base += nthreads * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int hb = base + u * nthreads;
      v[u] = hb < nhalves ? xv[hb] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int hb = base + u * nthreads;
      if (hb >= nhalves) continue;  // (both lanes of a pair alike: nhalves is even)
      float f[8];
      unpack_bf16x8(v[u], f);
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(f[e]));
      const float o = __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false));
      const BlockScale bs = block_scale(__builtin_fmaxf(a, o), qsc.den, qsc.rden, qsc.gs);
      const uint32_t word = __any(bs.code == kE4M3MaxCode) ? encode_half<true>(f, bs)
                                                           : encode_half<false>(f, bs);
      *(uint32_t*)&xq[4 * hb] = word;
      if ((hb & 1) == 0) xqs[hb >> 1] = (uint8_t)bs.code;
      if (store && fq.ws_packed != nullptr) {
        *(uint32_t*)(fq.ws_packed + 4 * (int64_t)hb) = word;
        if ((hb & 1) == 0) fq.ws_scales[hb >> 1] = (uint8_t)bs.code;
      }
    }
  }
}

// ---- small-M path: split K inside the workgroup -----------------------------------------
//
// For short activations (a few to a few hundred tokens) the tiled kernels leave most of
// the chip idle: M = 1 gives one tile row, so only N / 192 compute units work while the
// weights (the bulk of the bytes) stream through them. Here a workgroup owns A x B output
// blocks of 32 x 32 (32A weight rows, 32B activation rows) and its 4 waves split K:
// the 64-element chunks go in groups of four (one 128-byte line of codes per row), wave w
// taking groups w, w + 4, ..., so the waves move through K together.
// Each lane loads its fragments straight into registers (16 bytes = 32 codes of one row,
// the same K mapping as the LDS layouts of the tiled kernels), DG groups ahead of their
// use; the scales of a group come with one 16-byte load per row when K % 64 == 0
// (kVecScale: scale loads, which touch one cache line per row for a few bytes, had cost
// a third of the time at 256 rows), else two bytes per chunk. The four partial sums of
// each block meet in LDS at the end and are added in a fixed order.
//
// Requires K % 32 == 0, 16-byte aligned packed operands and 4-byte aligned scales, and
// both operands below 2^31 bytes (32-bit buffer offsets). In a last chunk that holds only
// 32 elements, the upper lane half reads past its row; its scale is forced to zero, so
// those products vanish (E2M1 codes are always finite).
//
// kFuse: the fused linear for the shortest activations (M * K <= kFuseElems). Once its
// first weight loads are in flight, the workgroup quantizes the M real activation rows
// together, two lanes per 16-element block exactly as the quantize kernel does (same functions, so the codes and
// scales are bit-identical to nvfp4_quantize's), into LDS in the NVFP4 layout; the
// workgroups of the first weight-row tile also store them to the caller's workspace.
// The K loop then reads the activation fragments from LDS (zeros for rows past M).
// Every workgroup along N repeats the quantization, which is why it is limited to a few
// thousand elements per thread block.
template <int A, int B, int DG, int NW, bool kFuse, bool kVecScale, bool kExp>
__global__ void __launch_bounds__(64 * NW) gemm_splitk_kernel(GemmProblem p, FusedQuant fq) {
  __shared__ float red[2][NW][16 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t xq[kFuse ? kFuseElems / 2 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t xqs[kFuse ? kFuseElems / 16 : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int tiles_m = (int)((p.M + 32 * B - 1) / (32 * B));
  const int tm = (int)blockIdx.x % tiles_m;  // consecutive workgroups share weight rows
  const int tn = (int)blockIdx.x / tiles_m;
  const int m0 = tm * 32 * B;
  const int n0 = tn * 32 * A;
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);
  const int nchunks = (int)((p.K + 63) / 64);
  // groups of four consecutive chunks (one 128-byte line of codes per row, and one
  // 16-byte load per row brings their scales); wave w takes groups w, w + NW, ...
  const int ngt = (nchunks + 3) / 4;
  const int ngroups = (ngt - wave + NW - 1) / NW;  // this wave's groups

  // Row windows [m0, M) and [n0, N) (see window_rsrc). Every load's per-lane offset holds
  // its row and its whole position along K: the upper lane half of a 32-element last
  // chunk reads past its row, which for the operand's last row is past its end, so that
  // position must be range-checked too. (The kFuse form reads no activations from memory
  // and never uses rxp or rxs.)
  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, m0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, m0, p.M, spitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);
  // lane's row r32 of 32-row group i of a window, its half h of a chunk: codes at
  // splitk_code_voff(i) + 32 c, two scale bytes at splitk_scale_voff(i) + 4 c
  auto splitk_code_voff = [&](int i) { return (uint32_t)(32 * i + r32) * pitch + (uint32_t)h * 16; };
  auto splitk_scale_voff = [&](int i) { return (uint32_t)(32 * i + r32) * spitch + (uint32_t)h * 2; };

  floatx16 acc[A][B];
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int g = 0; g < B; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  // ring slot s: the codes of a group's four chunks and its scales (kVecScale: the 16
  // scale bytes of the four chunks for the lane's row, both lane halves; otherwise the
  // lane's two bytes of chunk k in word k)
  u32x4 wraw[DG][4][A], xraw[DG][4][B];
  u32x4 wsv[DG][A], xsv[DG][B];
  // group G of this wave (chunks 4 (NW G + wave) .. + 3) into ring slot s
  auto load_group = [&](int s, int G) {
    const int c0 = 4 * (NW * G + wave);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (c0 + k < nchunks) {
        const int c = c0 + k;
#pragma unroll
        for (int i = 0; i < A; ++i) {
          wraw[s][k][i] = __builtin_amdgcn_raw_buffer_load_b128(
              rwp, (int)(splitk_code_voff(i) + (uint32_t)c * 32), 0, 0);
          if constexpr (!kVecScale)
            wsv[s][i][k] = __builtin_amdgcn_raw_buffer_load_b16(
                rws, (int)(splitk_scale_voff(i) + (uint32_t)c * 4), 0, 0);
        }
        if constexpr (!kFuse) {
#pragma unroll
          for (int g = 0; g < B; ++g) {
            xraw[s][k][g] = __builtin_amdgcn_raw_buffer_load_b128(
                rxp, (int)(splitk_code_voff(g) + (uint32_t)c * 32), 0, 0);
            if constexpr (!kVecScale)
              xsv[s][g][k] = __builtin_amdgcn_raw_buffer_load_b16(
                  rxs, (int)(splitk_scale_voff(g) + (uint32_t)c * 4), 0, 0);
          }
        }
      }
    }
    if constexpr (kVecScale) {
      // a whole group: its 16 scale bytes lie inside the row; a partial last group takes
      // 4 bytes per chunk instead (same layout), so no load reaches past the row's end
      auto vec = [&](__amdgpu_buffer_rsrc_t r, int grp) -> u32x4 {
        const uint32_t voff = (uint32_t)(32 * grp + r32) * spitch + (uint32_t)c0 * 4;
        if (c0 + 4 <= nchunks) return (u32x4)__builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
        u32x4 v{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c0 + k < nchunks) v[k] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(voff + 4 * k), 0, 0);
        return v;
      };
#pragma unroll
      for (int i = 0; i < A; ++i) wsv[s][i] = vec(rws, i);
      if constexpr (!kFuse) {
#pragma unroll
        for (int g = 0; g < B; ++g) xsv[s][g] = vec(rxs, g);
      }
    }
  };
  // chunk k of group G (ring slot s); the lane's two scale bytes sit in the low 16 bits
  auto compute = [&](int s, int G, int k) {
    const int c = 4 * (NW * G + wave) + k;
    // upper lane half of a 32-element last chunk: no elements, zero scale
    const bool dead = h == 1 && (int64_t)c * 64 + 32 >= p.K;
    auto lane_scales = [&](uint32_t v) { return kVecScale ? v >> (16 * h) : v; };
    u32x4 xr[B];
    uint32_t xs[B];
    if constexpr (kFuse) {
      // activation fragment from LDS (rows past M and the dead upper half read as zero)
      const bool live = r32 < p.M && !dead;
      xr[0] = live ? *(const u32x4*)&xq[r32 * pitch + (uint32_t)c * 32 + h * 16]
                   : u32x4{0u, 0u, 0u, 0u};
      xs[0] = live ? (uint32_t)*(const uint16_t*)&xqs[r32 * spitch + (uint32_t)c * 4 + h * 2]
                   : 0u;
    } else {
#pragma unroll
      for (int g = 0; g < B; ++g) {
        xr[g] = xraw[s][k][g];
        xs[g] = lane_scales(xsv[s][g][k]);
      }
    }
    half2_t wsc[A], xsc[B];
#pragma unroll
    for (int i = 0; i < A; ++i) wsc[i] = scales_to_f16<true>(dead ? 0u : lane_scales(wsv[s][i][k]));
#pragma unroll
    for (int g = 0; g < B; ++g) xsc[g] = scales_to_f16<true>(dead ? 0u : xs[g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t wf[A], xf[B];
#pragma unroll
      for (int i = 0; i < A; ++i) wf[i] = decode8<true>(wraw[s][k][i][j], j < 2 ? wsc[i].xx : wsc[i].yy);
#pragma unroll
      for (int g = 0; g < B; ++g) xf[g] = decode8<true>(xr[g][j], j < 2 ? xsc[g].xx : xsc[g].yy);
#pragma unroll
      for (int i = 0; i < A; ++i)
#pragma unroll
        for (int g = 0; g < B; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], xf[g], acc[i][g], 0, 0, 0);
      // keep each k-step's decode next to its MFMAs (bounded register use)
      __builtin_amdgcn_sched_barrier(0);
    }
  };


#pragma unroll
  for (int s = 0; s < DG; ++s)
    if (s < ngroups) load_group(s, s);
  // (after the first weight loads, so their latency overlaps the quantization)
  if constexpr (kFuse) {
    quantize_to_lds(fq, p.M, p.K, xq, xqs, tn == 0, 64 * NW);
    __syncthreads();
  }
  for (int G = 0; G < ngroups; G += DG) {
#pragma unroll
    for (int s = 0; s < DG; ++s) {
      if (G + s < ngroups) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (4 * (NW * (G + s) + wave) + k < nchunks) compute(s, G + s, k);
        if (G + s + DG < ngroups) load_group(s, G + s + DG);
      }
    }
  }

  // Partial sums: block by block, every wave writes its part, the owner wave (block
  // number % 4) adds the four in wave order, scales (apply_alpha) and stores.
  const bool n_vec = (p.N & 3) == 0;
  const Alpha alpha = gemm_alpha(p);
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int g = 0; g < B; ++g) {
      const int blk = i * B + g;
      float* rb = red[blk & 1][0];
#pragma unroll
      for (int v = 0; v < 16; ++v) rb[(wave * 16 + v) * 64 + lane] = acc[i][g][v];
      __syncthreads();
      if (wave == blk % NW) {
        const int64_t m = (int64_t)m0 + g * 32 + r32;
        if (m < p.M) {
          uint16_t* orow = p.out + m * p.N;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = (int64_t)n0 + i * 32 + 8 * q + 4 * h;
            float sv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * q + e;
              float s = rb[v * 64 + lane];
#pragma unroll
              for (int w = 1; w < NW; ++w) s += rb[(w * 16 + v) * 64 + lane];
              sv[e] = apply_alpha<kExp>(s, alpha);
            }
            const u32x2 b = bf16x4_rne(sv[0], sv[1], sv[2], sv[3]);
            if (n_vec && n + 3 < p.N) {
              *(u32x2*)&orow[n] = b;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < p.N) orow[n + e] = (uint16_t)(b[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    }
}

// ---- one to sixteen activation rows: weight rows spread over the whole chip ------------
//
// With a handful of activation rows the product is a read of the weights (1728 bytes per
// weight row at K = 3072) and takes the weight bytes over the load rate the workgroups
// reach. A compute unit loading 32 rows in 16-byte pieces, as the split-K kernel's
// register fragments do, gets about 15 GB/s there, and 32-row workgroups leave most of the
// chip idle at N = 3072 (96 of 256 compute units). Here a workgroup owns R <= 16 weight
// rows (a multiple of 4 the launcher picks so that the grid covers the chip: 12 rows, 256
// workgroups at N = 3072), its NW waves take the 256-element groups of K in turn (group g
// to wave g % NW; a group is one 128-byte line of codes and 16 scale bytes per row), and a
// 16 x 16 x 32 MFMA block holds the R weight rows against up to 16 activation rows.
//
// Lane (r, q) = (lane % 16, lane / 16) loads bytes 32q .. 32q + 31 of weight row r's line
// (elements 64q .. 64q + 63 of the group, four E4M3 blocks) with the row's scale bytes
// 4q .. 4q + 3, and the same of activation row r; lanes past the R weight rows or the M
// activation rows load nothing and hold zeros. MFMA 4h + j (h = 0, 1 the 16-byte half, j
// its 32-bit word) takes word j of half h from every lane: elements 64q + 32h + 8j .. + 7
// for q = 0..3, a reordering of the group's positions along K taken alike for both
// operands. The NW partial sums meet in LDS and are added in wave order.
//
// Requires M <= 16, K % 256 == 0, 16-byte aligned packed operands, 4-byte aligned scales,
// and both operands below 2^31 bytes (32-bit buffer offsets).
template <int NW, int DG, int B, bool kFuse, bool kExp>
__global__ void __launch_bounds__(64 * NW) gemm_gemv16_kernel(GemmProblem p, int R, FusedQuant fq) {
  typedef float floatx4 __attribute__((ext_vector_type(4)));
  __shared__ floatx4 red[NW][B][64];
  __shared__ __attribute__((aligned(16))) uint8_t xq[kFuse ? kFuseElemsGemv / 2 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t xqs[kFuse ? kFuseElemsGemv / 16 : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);
  const int ngt = (int)(p.K / 256);
  const int ng = (ngt - wave + NW - 1) / NW;  // this wave's groups: wave, wave + NW, ...
  // weight rows past N fall outside the window and read as zeros; rows of the next
  // workgroup (r >= R) and activation rows past M are not loaded
  const bool wlive = r < R;
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);
  const __amdgpu_buffer_rsrc_t rxp = window_rsrc(p.a_packed, 0, p.M, pitch);
  const __amdgpu_buffer_rsrc_t rxs = window_rsrc(p.a_scales, 0, p.M, spitch);

  // ring slot s: the lane's codes (two 16-byte halves) and four scale bytes of one group,
  // for its weight row and its activation rows r and 16 + r (kFuse: activations from LDS)
  u32x4 wc[DG][2], xc[DG][B][2];
  uint32_t wsv[DG], xsv[DG][B];
  auto load_x = [&](int s, int g) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int row = 16 * b + r;
      const bool live = row < p.M;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = gemv_code_voff(row, q, h, g, pitch);
        xc[s][b][h] = u32x4{0u, 0u, 0u, 0u};
        if (live) {
          if constexpr (kFuse) xc[s][b][h] = *(const u32x4*)&xq[off];
          else xc[s][b][h] = __builtin_amdgcn_raw_buffer_load_b128(rxp, (int)off, 0, 0);
        }
      }
      const uint32_t soff = gemv_scale_voff(row, q, g, spitch);
      xsv[s][b] = 0u;
      if (live) {
        if constexpr (kFuse) xsv[s][b] = *(const uint32_t*)&xqs[soff];
        else xsv[s][b] = __builtin_amdgcn_raw_buffer_load_b32(rxs, (int)soff, 0, 0);
      }
    }
  };
  auto load_w = [&](int s, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wc[s][h] = u32x4{0u, 0u, 0u, 0u};
      if (wlive)
        wc[s][h] = __builtin_amdgcn_raw_buffer_load_b128(rwp, (int)gemv_code_voff(r, q, h, g, pitch), 0, 0);
    }
    wsv[s] = 0u;
    if (wlive) wsv[s] = __builtin_amdgcn_raw_buffer_load_b32(rws, (int)gemv_scale_voff(r, q, g, spitch), 0, 0);
  };
  floatx4 acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // word j of half h spans elements 64q + 32h + 8j .. + 7: block 4q + 2h + j / 2, i.e.
  // byte 2h + j / 2 of the lane's scale word
  auto compute = [&](int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half2_t ws2 = scales_to_f16<true>(wsv[s] >> (16 * h));
      half2_t xs2[B];
#pragma unroll
      for (int b = 0; b < B; ++b) xs2[b] = scales_to_f16<true>(xsv[s][b] >> (16 * h));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t wf = decode8<true>(wc[s][h][j], j < 2 ? ws2.xx : ws2.yy);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const half8_t xf = decode8<true>(xc[s][b][h][j], j < 2 ? xs2[b].xx : xs2[b].yy);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf, acc[b], 0, 0, 0);
        }
      }
    }
  };

#pragma unroll
  for (int s = 0; s < DG; ++s)
    if (s < ng) load_w(s, wave + NW * s);
  if constexpr (kFuse) {
    // (after the first weight loads, so their latency overlaps the quantization)
    quantize_to_lds(fq, p.M, p.K, xq, xqs, blockIdx.x == 0, 64 * NW);
    __syncthreads();
  }
#pragma unroll
  for (int s = 0; s < DG; ++s)
    if (s < ng) load_x(s, wave + NW * s);
  for (int i = 0; i < ng; i += DG) {
#pragma unroll
    for (int s = 0; s < DG; ++s) {
      if (i + s < ng) {
        compute(s);
        if (i + s + DG < ng) {
          load_w(s, wave + NW * (i + s + DG));
          load_x(s, wave + NW * (i + s + DG));
        }
      }
    }
  }

  // lane (r, q) holds output rows 16b + r, columns n0 + 4q + {0..3} in acc[b]; wave 0
  // adds the NW parts in wave order, scales, rounds and stores them
#pragma unroll
  for (int b = 0; b < B; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  if (wave != 0) return;
  const int64_t n = n0 + 4 * q;
  if (4 * q >= R || n >= p.N) return;
  const Alpha alpha = gemm_alpha(p);
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const int64_t m = 16 * b + r;
    if (m >= p.M) continue;
    float tot[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) tot[e] = red[0][b][lane][e];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const floatx4 part = red[w][b][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[e] += part[e];
    }
    float sv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = apply_alpha<kExp>(tot[e], alpha);
    const u32x2 bits = bf16x4_rne(sv[0], sv[1], sv[2], sv[3]);
    uint16_t* orow = p.out + m * p.N;
    if ((p.N & 3) == 0 && n + 3 < p.N) {
      *(u32x2*)&orow[n] = bits;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) orow[n + e] = (uint16_t)(bits[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Device-resident global scales (whose product the launch cannot see) and host pairs
// whose product is not a normal fp32 run the tiled kernels' ldexp epilogue (apply_alpha).
bool alpha_needs_exp(const GemmProblem& p) { return p.a_gs_dev != nullptr || p.alpha_exp != 0; }

template <int BM, int BN, int KC, int WM, int WN>
hipError_t launch_tile(const GemmProblem& p, hipStream_t stream, bool fast) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles);
  const bool ext = alpha_needs_exp(p);
  if (fast && ext)
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, true>), grid, dim3(256), 0, stream, p);
  else if (fast)
    hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, false>), grid, dim3(256), 0, stream, p);
  else if (ext)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, KC, WM, WN, true, false, true>), grid,
                       dim3(64 * WM * WN), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, KC, WM, WN, true, false, false>), grid,
                       dim3(64 * WM * WN), 0, stream, p);
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

// The epilogues' packed fp32 -> bf16 conversion against the bit-pattern rounding on
// every binary32 pattern except NaN: pattern u in the low half, u ^ 0x00010000 (its
// neighbour two bf16 ulps away in the other rounding direction's parity) in the high
// half, so both halves of the instruction see every pattern.
__global__ void selftest_bf16_exhaustive_kernel(unsigned long long* __restrict__ count,
                                                uint32_t* __restrict__ first) {
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t nthreads = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u = tid; u < (1ull << 32); u += nthreads) {
    const uint32_t lo = (uint32_t)u, hi = lo ^ 0x00010000u;
    const float a = u2f(lo), b = u2f(hi);
    if (a != a || b != b) continue;
    const uint32_t hw = bf16x2_rne(a, b);
    const uint32_t sw = bf16_rne(a) | (bf16_rne(b) << 16);
    if (hw != sw) {
      const unsigned long long k = atomicAdd(count, 1ull);
      if (k < 16) first[k] = lo;
    }
  }
}

// Rough cost model (core cycles of one launch) used to choose between the kernels; the
// 32x32x16 f16 MFMA issues every ~34 cycles back to back and slows by ~5.5 cycles per
// VALU instruction beyond about 3 per MFMA (the decode costs 8 VALU per fragment of 8
// elements per lane), a slope fitted to the 128 x 64 / 128 x 128 / 128 x 192 tiles'
// measured times; the split-K costs are its own measurements.
#ifndef NVFP4_GEMM_KC
#define NVFP4_GEMM_KC 2
#endif
#ifndef NVFP4_GEMM_WM
#define NVFP4_GEMM_WM 2
#endif
#ifndef NVFP4_GEMM_WN
#define NVFP4_GEMM_WN 2
#endif
#ifndef NVFP4_FIT_BM
#define NVFP4_FIT_BM 288
#define NVFP4_FIT_BN 192
#endif
constexpr int kTileBM = 256, kTileBN = 256, kTileKC = NVFP4_GEMM_KC;
constexpr int kFitBM = NVFP4_FIT_BM, kFitBN = NVFP4_FIT_BN;

double mfma_cycles(double frags_per_mfma) {
  const double v = 8.0 * frags_per_mfma;
  return 34.0 + (v > 3.0 ? 5.5 * (v - 3.0) : 0.0);
}
int64_t passes(int64_t wgs, int64_t cus) { return (wgs + cus - 1) / cus; }

// Split-K workgroup shape for M activation rows: 32 x 32B outputs with B the smallest
// of 1, 2, 4 that covers min(M, 128) rows (measured: wider shapes do not pay at these M).
SplitShape splitk_shape(int64_t M) {
  if (M <= 32) return {1, 1};
  if (M <= 64) return {1, 2};
  return {1, 4};
}

template <int A, int B, int DG, int NW, bool kFuse, bool kVecScale>
void launch_splitk_kernel(dim3 grid, dim3 block, hipStream_t stream, const GemmProblem& p,
                          const FusedQuant& fq) {
  if (alpha_needs_exp(p))
    hipLaunchKernelGGL((gemm_splitk_kernel<A, B, DG, NW, kFuse, kVecScale, true>), grid, block, 0,
                       stream, p, fq);
  else
    hipLaunchKernelGGL((gemm_splitk_kernel<A, B, DG, NW, kFuse, kVecScale, false>), grid, block, 0,
                       stream, p, fq);
}

hipError_t launch_splitk(const GemmProblem& p, hipStream_t stream, SplitShape s) {
  const int64_t wgs = ((p.N + 32 * s.a - 1) / (32 * s.a)) * ((p.M + 32 * s.b - 1) / (32 * s.b));
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  constexpr int NW = 4;  // 8 or 16 waves per workgroup measured no faster
  const dim3 grid((unsigned)wgs), block(64 * NW);
  const FusedQuant none{};
  // 16-byte scale loads need 4-byte aligned scale rows (K % 64 == 0)
  // groups in flight per wave by workgroup shape (registers: about 40 VGPRs per group
  // and activation group); measured: deeper rings gain nothing
  if (p.K % 64 == 0) {
    if (s.b == 1) launch_splitk_kernel<1, 1, 4, NW, false, true>(grid, block, stream, p, none);
    else if (s.b == 2) launch_splitk_kernel<1, 2, 3, NW, false, true>(grid, block, stream, p, none);
    else launch_splitk_kernel<1, 4, 2, NW, false, true>(grid, block, stream, p, none);
  } else {
    if (s.b == 1) launch_splitk_kernel<1, 1, 4, NW, false, false>(grid, block, stream, p, none);
    else if (s.b == 2) launch_splitk_kernel<1, 2, 3, NW, false, false>(grid, block, stream, p, none);
    else launch_splitk_kernel<1, 4, 2, NW, false, false>(grid, block, stream, p, none);
  }
  return hipGetLastError();
}

template <int NW, int B, bool kFuse>
void launch_gemv16_kernel(const GemmProblem& p, const FusedQuant& fq, hipStream_t stream,
                          unsigned wgs, int R) {
  if (alpha_needs_exp(p))
    hipLaunchKernelGGL((gemm_gemv16_kernel<NW, 4, B, kFuse, true>), dim3(wgs), dim3(64 * NW), 0,
                       stream, p, R, fq);
  else
    hipLaunchKernelGGL((gemm_gemv16_kernel<NW, 4, B, kFuse, false>), dim3(wgs), dim3(64 * NW), 0,
                       stream, p, R, fq);
}

template <bool kFuse>
hipError_t launch_gemv16(const GemmProblem& p, const FusedQuant& fq, hipStream_t stream, int64_t cus) {
  const int R = gemv16_rows(p.N, cus > 0 ? cus : 256);
  const int64_t wgs = (p.N + R - 1) / R;
  if (wgs > 0x7FFFFFFF || p.M > 32 || p.K % 256 != 0) return hipErrorInvalidValue;
  if (kFuse && p.M * p.K > kFuseElemsGemv) return hipErrorInvalidValue;
  // eight waves once K has eight groups (more loads in flight per compute unit); one or
  // two 16-row activation blocks
  const bool wide = p.K / 256 >= 8;
  if (p.M <= 16) {
    if (wide) launch_gemv16_kernel<8, 1, kFuse>(p, fq, stream, (unsigned)wgs, R);
    else launch_gemv16_kernel<4, 1, kFuse>(p, fq, stream, (unsigned)wgs, R);
  } else {
    if (wide) launch_gemv16_kernel<8, 2, kFuse>(p, fq, stream, (unsigned)wgs, R);
    else launch_gemv16_kernel<4, 2, kFuse>(p, fq, stream, (unsigned)wgs, R);
  }
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool aligned, int64_t cus, bool allow_gemv16) {
  constexpr int BM = kTileBM, BN = kTileBN, KC = kTileKC;
  constexpr int FBM = kFitBM, FBN = kFitBN;
  GemmPlan plan{};
  cus = cus > 0 ? cus : 256;
  // 32-bit buffer offsets (with one tile of rows past the end) for the 256x256, fit and
  // split-K kernels
  const bool fits32 = fits_i31(M + FBM, K / 2) && fits_i31(N + FBN, K / 2);
  const bool fits32_256 = fits_i31(M + BM, K / 2) && fits_i31(N + BN, K / 2);
  const bool fast = aligned && (K % (64 * KC) == 0) && fits32_256;
  const int64_t nk = K / 128;
  // tiled kernels: one tile per compute unit at a time, plus epilogue and prologue
  const int64_t t256 = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t tfit = ((M + FBM - 1) / FBM) * ((N + FBN - 1) / FBN);
  const double c256 = fast ? (double)passes(t256, cus) * (nk * 128 * mfma_cycles(0.5) + 20000.0) : 1e300;
  const bool fit_ok = aligned && K % 128 == 0 && fits32;
  const double cfit = fit_ok ? (double)passes(tfit, cus) * (nk * 108 * mfma_cycles(7.5 / 13.5) + 20000.0) : 1e300;
  // 128 x 192 tiles (2 x 3 blocks per wave: more decode per MFMA, but 4x the tiles of
  // 256 x 256) for activations too short to fill the chip with the larger tiles
  const int64_t t128 = ((M + 127) / 128) * ((N + 191) / 192);
  const double c128 = fast ? (double)passes(t128, cus) * (nk * 48 * mfma_cycles(5.0 / 6.0) + 20000.0) : 1e300;
  // 128 x 128 tiles (2 x 2 blocks per wave, one fragment decoded per MFMA): the most
  // tiles, for activations of a few hundred rows or a few hundred x wide weights
  const int64_t t128sq = ((M + 127) / 128) * ((N + 127) / 128);
  const double c128sq = fast ? (double)passes(t128sq, cus) * (nk * 32 * mfma_cycles(1.0) + 20000.0) : 1e300;
  // 128 x 64 tiles (2 x 1 blocks per wave, 1.5 fragments per MFMA): shorter tiles still
  const int64_t t12864 = ((M + 127) / 128) * ((N + 63) / 64);
  const double c12864 = fast ? (double)passes(t12864, cus) * (nk * 16 * mfma_cycles(1.5) + 20000.0) : 1e300;
  // Split K inside the workgroup (short activations, at most 512 rows: it reads the
  // activations once per 32 weight rows, which stops paying beyond that). Measured cost,
  // in the units of the tile costs above (the 128 x 128 tile's): ~6000 cycles of launch
  // and reduction plus, per pass over the chip, 680 / 1110 / 2000 per 128 elements of K
  // for 32-row groups B = 1 / 2 / 4 per workgroup (M = 17, 64 and 256 at K = 3072,
  // against the double-stage tiles).
  const bool split_ok = aligned && K % 32 == 0 && fits32;
  const SplitShape sh = splitk_shape(M);
  const int64_t wsplit = ((N + 31) / 32) * ((M + 32 * sh.b - 1) / (32 * sh.b));
  const double csplit = 6000.0 + (double)passes(wsplit, cus) * ((double)K / 128.0) *
                                     (sh.b == 1 ? 680.0 : sh.b == 2 ? 1110.0 : 2000.0);
  // 64 x 64 tiles whose waves split K, in one pass over the chip only (a second pass of
  // these long per-tile runs loses to the larger tiles). Measured at N = 3072 and 12288,
  // K = 3072 and 12288: one pass takes about 4.7 us plus 0.19 us per 128 elements of K,
  // here in the units of the 128 x 64 tile's cost (16.2 us at 256 x 3072 x 3072).
  const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
  const bool ws_ok = aligned && K % 512 == 0 && fits_i31(M + 64, K / 2) && fits_i31(N + 64, K / 2) &&
                     t64 <= cus;
  const double cws = ws_ok ? (double)nk * 624.0 + 15200.0 : 1e300;
  // 128 x 128 tiles, two row bands of two waves splitting K: 0.75 fragments per MFMA
  // against the 128 x 128 tile's 1, for a larger reduction at the end; one pass only.
  // Measured at 1000 x 3072 (K = 3072, 6144, 12288): 22.9 / 37.5 / 68.9 us against the
  // 128 x 128 tile's 21.9 / 40.7 / 77.1 (here 1620 per stage plus 31 400).
  const bool ws2_ok = aligned && K % 256 == 0 && fits_i31(M + 128, K / 2) && fits_i31(N + 128, K / 2) &&
                      t128sq <= cus;
  const double cws2 = ws2_ok ? (double)nk * 1620.0 + 31400.0 : 1e300;
  plan.kernel = fast ? NVFP4_GEMM_TILE256 : NVFP4_GEMM_GENERIC;
  plan.split = splitk_shape(M);
  if (fast || fit_ok) {
    double best = c256;
    if (fit_ok && cfit <= best) { plan.kernel = NVFP4_GEMM_FIT; best = cfit; }
    if (fast && c128 < best) { plan.kernel = NVFP4_GEMM_TILE128; best = c128; }
    if (fast && c128sq < best) { plan.kernel = NVFP4_GEMM_TILE128X128; best = c128sq; }
    if (fast && c12864 < best) { plan.kernel = NVFP4_GEMM_TILE128X64; best = c12864; }
    if (cws < best) { plan.kernel = NVFP4_GEMM_WSPLIT64; best = cws; }
    if (cws2 < best) { plan.kernel = NVFP4_GEMM_WSPLIT128; best = cws2; }
    if (split_ok && M <= 512 && csplit < best) plan.kernel = NVFP4_GEMM_SPLITK;
    // at most 16 activation rows, or up to 32 while 16-row workgroups fit one pass over the
    // compute units (two activation blocks hold one 512-thread workgroup per compute unit,
    // so more passes cost a whole workgroup's latency each; 17 x 18432 x 3072: 20.9 us
    // against split-K's 13.7): the weights' read, spread over the whole chip
    const bool gemv_rows = M <= 16 || (M <= 32 && (N + 15) / 16 <= cus);
    if (allow_gemv16 && gemv_rows && K % 256 == 0 && fits_i31(M + 32, K / 2) && fits_i31(N + 16, K / 2))
      plan.kernel = NVFP4_GEMM_GEMV16;
  } else if (split_ok && M <= 512 && tfit * 4 <= cus) {
    // against the register-staged kernel (K % 128 != 0): few tiles only
    plan.kernel = NVFP4_GEMM_SPLITK;
  }
  return plan;
}

template <int BM, int BN, int KS>
hipError_t launch_wsplit(const GemmProblem& p, hipStream_t stream) {
  const int64_t t = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (t > 0x7FFFFFFF || p.K % (128 * KS) != 0) return hipErrorInvalidValue;
  if (alpha_needs_exp(p))
    hipLaunchKernelGGL((gemm_wsplit_kernel<BM, BN, KS, true>), dim3((unsigned)t), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_wsplit_kernel<BM, BN, KS, false>), dim3((unsigned)t), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev) {
  const bool aligned = ((uintptr_t)p.a_packed % 16 == 0) && ((uintptr_t)p.w_packed % 16 == 0) &&
                       ((uintptr_t)p.a_scales % 4 == 0) && ((uintptr_t)p.w_scales % 4 == 0);
  const GemmPlan plan = plan_gemm(p.M, p.N, p.K, aligned, dev.num_cus);
  switch (plan.kernel) {
    case NVFP4_GEMM_SPLITK:
      return launch_splitk(p, stream, plan.split);
    case NVFP4_GEMM_GEMV16:
      return launch_gemv16<false>(p, FusedQuant{}, stream, dev.num_cus);
    case NVFP4_GEMM_FIT: {
      const int64_t tfit = ((p.M + kFitBM - 1) / kFitBM) * ((p.N + kFitBN - 1) / kFitBN);
      if (tfit > 0x7FFFFFFF) return hipErrorInvalidValue;
      if (alpha_needs_exp(p))
        hipLaunchKernelGGL((gemm_fit_kernel<kFitBM, kFitBN, true>), dim3((unsigned)tfit), dim3(256),
                           0, stream, p);
      else
        hipLaunchKernelGGL((gemm_fit_kernel<kFitBM, kFitBN, false>), dim3((unsigned)tfit), dim3(256),
                           0, stream, p);
      return hipGetLastError();
    }
    case NVFP4_GEMM_TILE128: {
      const int64_t t = ((p.M + 127) / 128) * ((p.N + 191) / 192);
      if (t > 0x7FFFFFFF) return hipErrorInvalidValue;
      if (alpha_needs_exp(p))
        hipLaunchKernelGGL((gemm_dma_kernel<128, 192, true>), dim3((unsigned)t), dim3(256), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((gemm_dma_kernel<128, 192, false>), dim3((unsigned)t), dim3(256), 0,
                           stream, p);
      return hipGetLastError();
    }
    case NVFP4_GEMM_TILE128X128: {
      const int64_t t = ((p.M + 127) / 128) * ((p.N + 127) / 128);
      if (t > 0x7FFFFFFF) return hipErrorInvalidValue;
      if (alpha_needs_exp(p))
        hipLaunchKernelGGL((gemm_dma_kernel<128, 128, true>), dim3((unsigned)t), dim3(256), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((gemm_dma_kernel<128, 128, false>), dim3((unsigned)t), dim3(256), 0,
                           stream, p);
      return hipGetLastError();
    }
    case NVFP4_GEMM_TILE128X64: {
      const int64_t t = ((p.M + 127) / 128) * ((p.N + 63) / 64);
      if (t > 0x7FFFFFFF) return hipErrorInvalidValue;
      if (alpha_needs_exp(p))
        hipLaunchKernelGGL((gemm_dma_kernel<128, 64, true>), dim3((unsigned)t), dim3(256), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((gemm_dma_kernel<128, 64, false>), dim3((unsigned)t), dim3(256), 0,
                           stream, p);
      return hipGetLastError();
    }
    case NVFP4_GEMM_WSPLIT64:
      return launch_wsplit<64, 64, 4>(p, stream);
    case NVFP4_GEMM_WSPLIT128:
      return launch_wsplit<128, 128, 2>(p, stream);
    default:
      return launch_tile<kTileBM, kTileBN, kTileKC, NVFP4_GEMM_WM, NVFP4_GEMM_WN>(
          p, stream, plan.kernel == NVFP4_GEMM_TILE256);
  }
}

bool linear_fused(int64_t M, int64_t N, int64_t K, bool aligned, int64_t cus) {
  // activations small enough to quantize in every workgroup (and to sit in its LDS), on
  // the GEMM the product would run: the 16-row kernel (up to 24576 elements: its loads of
  // the weights are in flight meanwhile; at K = 3072 the fused form took 4.3, 5.6 and
  // 6.8 us for 1, 6 and 10 rows, the quantize kernel and the GEMM 6.4 us for 11 rows) or
  // split-K with one 32-row activation group (up to 16384)
  if (M > 32) return false;
  const GemmPlan g = plan_gemm(M, N, K, aligned, cus);
  if (g.kernel == NVFP4_GEMM_GEMV16) return M * K <= kFuseElemsGemv;
  return g.kernel == NVFP4_GEMM_SPLITK && M * K <= kFuseElems;
}

hipError_t launch_linear_fused(const GemmProblem& p, const FusedQuant& fq, hipStream_t stream,
                               int64_t cus) {
  if (p.M > 32) return hipErrorInvalidValue;
  // (the entry points have checked the operands' alignment, as linear_fused assumes)
  if (plan_gemm(p.M, p.N, p.K, true, cus).kernel == NVFP4_GEMM_GEMV16)
    return launch_gemv16<true>(p, fq, stream, cus);
  const int64_t wgs = (p.N + 31) / 32;
  if (p.M * p.K > kFuseElems || wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (p.K % 64 == 0)
    launch_splitk_kernel<1, 1, 4, 4, true, true>(dim3((unsigned)wgs), dim3(256), stream, p, fq);
  else
    launch_splitk_kernel<1, 1, 4, 4, true, false>(dim3((unsigned)wgs), dim3(256), stream, p, fq);
  return hipGetLastError();
}

hipError_t launch_selftest_bf16_exhaustive(unsigned long long* count, uint32_t* first,
                                           hipStream_t stream) {
  hipLaunchKernelGGL(selftest_bf16_exhaustive_kernel, dim3(8192), dim3(256), 0, stream, count,
                     first);
  return hipGetLastError();
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
