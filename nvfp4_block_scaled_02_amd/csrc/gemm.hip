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
//  * Packed 4-bit tiles and scale bytes stream from HBM into LDS (four stage buffers in
//    the direct-to-LDS kernels, two in the register-staged one); decode happens in
//    registers right before the MFMA, so LDS holds 4-bit data and its traffic stays 4x
//    below an f16-staged design.
//  * LDS layout of a packed tile: a lane reads its operand fragment for a 64-element
//    chunk (row r, bytes [16h, 16h+16) of the chunk) with one 16-byte LDS load, free of
//    bank conflicts. The direct-to-LDS kernels (288 x 192, 256 x 256, 128 x 192, 128 x 128
//    and 128 x 64 tiles) keep each row's 64 bytes of a stage together in 1 KiB pieces of 16 rows with the 16-byte
//    chunks swizzled (chunk_swz), because their loads read whole 64-byte row segments;
//    the register-staged kernel stores 64 slots of 16 bytes per 32-row group and chunk
//    in MFMA lane order.
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
//    binary32 range), round to nearest even bf16. The direct-to-LDS kernels pass each
//    32-row group of a wave's blocks through LDS and store 16-byte row pieces; the
//    others store each lane's 8 bytes directly.
//  * Short activations (split-K kernel): K is split over the waves of a workgroup and
//    the partial sums meet in LDS; nvfp4_linear's fused form quantizes the activations
//    into LDS first.
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

// ---- 256 x 256 and 128 x 192 tiles: direct-to-LDS loads, four code stages, one pipeline
// across stages ----
//
// 2 x 2 waves of BM/2 x BN/2: 4 x 4 blocks of 32 x 32 for 256 x 256 (the large-M tile),
// 2 x 3 for 128 x 192, 2 x 2 for 128 x 128 and 2 x 1 for 128 x 64 (medium M: more tiles,
// so fewer rows still fill the chip, at a higher decode cost per MFMA). Loads, LDS image and stage pipeline
// are the fit kernel's (below): code loads of 16 rows x the stage's 64 bytes (4 lanes per
// row) into 1 KiB pieces whose 16-byte chunks are swizzled by chunk_swz, scale loads of
// 64 rows x 16 bytes (a pair of stages) into three pair buffers, four code buffers filled
// three stages ahead, one wait and barrier per stage; range-checked buffer loads, so a
// ragged tile needs no clamping. 4 x 32 KiB + 3 x 8 KiB = 152 KiB of LDS at 256 x 256,
// 4 x 20 KiB + 3 x 5 KiB = 95 KiB at 128 x 192.
template <int BM, int BN>
struct alignas(16) GemmSmem256 {
  uint8_t x[4][BM * 64];
  uint8_t w[4][BN * 64];
  uint8_t sc[3][(BM + BN) * 16];
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
  constexpr int kPa = BM / 16, kPw = BN / 16;
  static_assert(kPa % NW == 0 && kPw % NW == 0, "code pieces divide among waves");
  constexpr int kPaW = kPa / NW, kPwW = kPw / NW;
  constexpr int kSx = BM / 64;
  constexpr int kSp = kSx + BN / 64;  // scale pieces per pair of stages
  static_assert(BM % 64 == 0 && BN % 64 == 0 && kSp <= 2 * NW, "one scale load per wave and stage");
  constexpr int kLoadsPerWave = kPaW + kPwW + 1;
  static_assert(kLoadsPerWave < 16, "one stage of loads fits the vmcnt immediate");
  constexpr int kLoadsPerStep = (kLoadsPerWave + kSteps - 3) / (kSteps - 2);

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
  const int nk = (int)(p.K / 128);
  const int npair = (nk + 1) >> 1;
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);

  const __amdgpu_buffer_rsrc_t rxp = make_rsrc(p.a_packed, (uint32_t)p.M * pitch);
  const __amdgpu_buffer_rsrc_t rwp = make_rsrc(p.w_packed, (uint32_t)p.N * pitch);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.a_scales, (uint32_t)p.M * spitch);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.w_scales, (uint32_t)p.N * spitch);
  const int lr = lane >> 2;
  const uint32_t voff_p = lr * pitch + 16 * ((lane & 3) ^ chunk_swz(lr));
  const uint32_t voff_s = lane * spitch;

  // scale piece half * NW + wave of a pair (slots past the last piece repeat it, writing
  // the same bytes to the same place)
  auto issue_scale = [&](int pair, int half, int sb) {
    const int i = min(half * NW + wave, kSp - 1);
    const bool isx = i < kSx;
    const uint32_t row = isx ? (uint32_t)(m0 + 64 * i) : (uint32_t)(n0 + 64 * (i - kSx));
    buffer_load_lds16(isx ? rxs : rws, &sm.sc[sb][i * 1024], voff_s, row * spitch + (uint32_t)pair * 16);
  };
  auto issue = [&](int j, int stage, int buf, int t, int spair, int sb) {
    if (j < kPaW) {
      const int i = j * NW + wave;
      buffer_load_lds16(rxp, &sm.x[buf][i * 1024], voff_p,
                        (uint32_t)(m0 + 16 * i) * pitch + (uint32_t)stage * 64);
    } else if (j < kPaW + kPwW) {
      const int i = (j - kPaW) * NW + wave;
      buffer_load_lds16(rwp, &sm.w[buf][i * 1024], voff_p,
                        (uint32_t)(n0 + 16 * i) * pitch + (uint32_t)stage * 64);
    } else {
      issue_scale(spair, t & 1, sb);
    }
  };

  floatx16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  // fragments of two chunks (by chunk order) and decoded operands of two k-steps
  const int fr0 = (r32 >> 4) * 1024 + (r32 & 15) * 64 + 16 * (h ^ chunk_swz(r32 & 15));
  const int wfrag = wave_n * FN * 2048;
  const int xfrag = wave_m * FM * 2048;
  const int wsw = (BM + wave_n * WTN + r32) * 16 + 2 * h;
  const int xsw = (wave_m * WTM + r32) * 16 + 2 * h;
  u32x4 wraw[2][FN], xraw[2][FM];
  uint32_t wsr[2][FN], xsr[2][FM];
  half2_t wsc[FN], xsc[FM];
  half8_t wf[2][FN], xf[2][FM];
  auto read_chunk = [&](int par, int buf, int c, int sb, int sub) {
    const int fr = fr0 ^ (32 * c);
    const uint8_t* wb = &sm.w[buf][wfrag + fr];
    const uint8_t* xb = &sm.x[buf][xfrag + fr];
    const uint8_t* scb = &sm.sc[sb][sub * 8 + c * 4];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[par][i] = *(const u32x4*)(wb + i * 2048);
      wsr[par][i] = *(const uint16_t*)(scb + wsw + i * 512);
    }
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      xraw[par][g] = *(const u32x4*)(xb + g * 2048);
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

  // prologue: scales of pairs 0 and 1, codes of stages 0, 1 and 2
  issue_scale(0, 0, 0);
  issue_scale(0, 1, 0);
  issue_scale(npair > 1 ? 1 : 0, 0, 1);
  issue_scale(npair > 1 ? 1 : 0, 1, 1);
#pragma unroll
  for (int j = 0; j < kPaW + kPwW; ++j) issue(j, 0, 0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < kPaW + kPwW; ++j) issue(j, nk > 1 ? 1 : nk - 1, 1, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < kPaW + kPwW; ++j) issue(j, nk > 2 ? 2 : nk - 1, 2, 0, 0, 0);
  // stages 0 and 1 (stage 0 reads stage 1's first chunk ahead); stage 2's loads may
  // still be in flight: the wait at the end of stage 0 covers them
  wait_vmcnt<kPaW + kPwW>();
  __builtin_amdgcn_s_barrier();
  read_chunk(0, 0, 0, 0, 0);
  decode_step(0, 0, wf[0], xf[0]);

  constexpr int kMfmaPerStep = FN * FM;
  constexpr int kReadsPerChunk = 2 * (FN + FM);
  int buf = 0;
  for (int t = 0; t < nk; ++t) {
    const int nbuf = (buf + 1) & 3;  // stage t + 1 (complete since the end of stage t - 1)
    const int lbuf = (buf + 3) & 3;  // stage t + 3 (its buffer held stage t - 1)
    const int lstage = t + 3 < nk ? t + 3 : nk - 1;
    const int pair = t >> 1;
    const int sb = pair % 3, sbn = ((t + 1) >> 1) % 3;
    const int spair = pair + 2 < npair ? pair + 2 : npair - 1;
    const int sbl = (pair + 2) % 3;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int cur = st & 1;
      const int chunk = st >> 2, j = st & 3;
#pragma unroll
      for (int l = 0; l < kLoadsPerStep; ++l)
        if (st * kLoadsPerStep + l < kLoadsPerWave) issue(st * kLoadsPerStep + l, lstage, lbuf, t, spair, sbl);
      const bool reads = j == 0;
      if (reads) {  // next chunk: the second of this stage, then the first of the next
        if (chunk == 0) read_chunk(1, buf, 1, sb, t & 1);
        else read_chunk(0, nbuf, 0, sbn, (t + 1) & 1);
      }
      // decode of the next k-step (the first k-step of the next stage after the last)
      if (st + 1 < kSteps) decode_step((st + 1) >> 2 & 1, (st + 1) & 3, wf[cur ^ 1], xf[cur ^ 1]);
      else decode_step(0, 0, wf[cur ^ 1], xf[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < kMfmaPerStep; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (reads && q < kReadsPerChunk) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        if (q < kLoadsPerStep && st * kLoadsPerStep + q < kLoadsPerWave)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS
        __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_GEMM_VALU_PER_MFMA, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<kLoadsPerWave>();
    __builtin_amdgcn_s_barrier();
    buf = nbuf;
  }

  // drain the last (unused) loads before the stage buffers stage the stores
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  store_tile_lds<FM, FN, false, kExp>(acc, p, gemm_alpha(p), (int64_t)m0 + wave_m * WTM,
                                      (int64_t)n0 + wave_n * WTN, lane,
                                      (uint16_t*)&sm.x[0][0] + wave * 32 * kStoreRowPad(FN));
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
// than by its bytes, so a code load reads whole 64-byte row segments (16 rows x the
// stage's 64 bytes, 4 lanes per row) and a scale load 64 rows x 16 bytes (the scales of
// two stages).
//
// LDS image of a stage: per 16-row piece 1 KiB, row r's 64 bytes (chunk 0, then chunk 1)
// at 64 r, its 16-byte pieces q = 2 * chunk + half swizzled to slot q ^ chunk_swz(r).
// Scales: 16 bytes per row for a pair of stages, activation rows (rounded up to whole
// 64-row pieces) first, then weight rows; three pair buffers.
template <int BM, int BN>
struct alignas(16) GemmSmemFit {
  static constexpr int kScaleRowsX = (BM + 63) / 64 * 64;
  uint8_t x[4][BM * 64];  // activations: [stage buffer][16-row piece]
  uint8_t w[4][BN * 64];  // weights
  uint8_t sc[3][(kScaleRowsX + BN) * 16];  // scale bytes: [pair buffer][row][16]
};

// Requires K % 128 == 0, 16-byte aligned packed operands, 4-byte aligned scales, and
// (rows + one tile) x K/2 below 2^31 for both operands (32-bit buffer offsets).
//
// Stage t lives in LDS buffer t % 4; its loads are issued during stage t-3, spread over
// the first k-steps. At the end of stage t each wave waits until every load it issued
// before stage t has landed (stages up to t+2; those for t+3 stay in flight) and the
// workgroup meets at a barrier. So stage t+1 is complete in LDS throughout stage t, whose
// second chunk reads stage t+1's first chunk and decodes its first k-step; and by the
// barrier every wave has consumed its reads of stage t, whose buffer the loads issued
// during stage t+1 overwrite. The scales of stage pair u (stages 2u, 2u+1) live in pair
// buffer u % 3 and are loaded during stages 2u-4 and 2u-3 (one load per wave each), so
// they are complete before stage 2u-1 first reads them, and their buffer's previous pair
// was last read in stage 2u-5.
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

  // Loads per stage: one 16-byte load per lane fills a 16-row code piece of 1 KiB. Two
  // lists (packed x, packed w); wave w takes entries j * NW + w of each. Every wave issues
  // the same number of loads, so the vmcnt wait counts the same; entries past a list
  // repeat its last one, which writes the same bytes to the same place. Plus one scale
  // load per wave: a pair's 2 * NW scale pieces (64 rows x 16 bytes) over its two stages.
  constexpr int kPa = BM / 16, kPw = BN / 16;
  constexpr int kPaW = (kPa + NW - 1) / NW, kPwW = (kPw + NW - 1) / NW;
  constexpr int kRowsSx = GemmSmemFit<BM, BN>::kScaleRowsX;
  constexpr int kSx = kRowsSx / 64;
  static_assert(BN % 64 == 0 && kSx + BN / 64 == 2 * NW, "one scale load per wave and stage");
  constexpr int kLoadsPerWave = kPaW + kPwW + 1;
  static_assert(kLoadsPerWave < 16, "one stage of loads fits the vmcnt immediate");
  constexpr int kLoadsPerStep = (kLoadsPerWave + kSteps - 3) / (kSteps - 2);

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
  const int nk = (int)(p.K / 128);
  const int npair = (nk + 1) >> 1;
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);

  // Buffer resources: the range check returns zeros for rows past M (or N), so a ragged
  // last tile needs no clamping.
  const __amdgpu_buffer_rsrc_t rxp = make_rsrc(p.a_packed, (uint32_t)p.M * pitch);
  const __amdgpu_buffer_rsrc_t rwp = make_rsrc(p.w_packed, (uint32_t)p.N * pitch);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.a_scales, (uint32_t)p.M * spitch);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.w_scales, (uint32_t)p.N * spitch);
  const int lr = lane >> 2;  // row of a code piece this lane loads
  const uint32_t voff_p = lr * pitch + 16 * ((lane & 3) ^ chunk_swz(lr));
  const uint32_t voff_s = lane * spitch;

  // Scale piece `half` * NW + wave of stage pair `pair` into pair buffer `sb`; pieces below
  // kSx hold activation rows, the rest weight rows (selects, no branch).
  auto issue_scale = [&](int pair, int half, int sb) {
    const int i = half * NW + wave;
    const bool isx = i < kSx;
    const uint32_t row = isx ? (uint32_t)(m0 + 64 * i) : (uint32_t)(n0 + 64 * (i - kSx));
    buffer_load_lds16(isx ? rxs : rws, &sm.sc[sb][i * 1024], voff_s, row * spitch + (uint32_t)pair * 16);
  };
  // Load j of this wave in stage t: code pieces of stage `stage` into buffer `buf`, the
  // last one the stage's scale piece (pair `spair` into pair buffer `sb`).
  auto issue = [&](int j, int stage, int buf, int t, int spair, int sb) {
    if (j < kPaW) {
      const int i = min(j * NW + wave, kPa - 1);
      buffer_load_lds16(rxp, &sm.x[buf][i * 1024], voff_p,
                        (uint32_t)(m0 + 16 * i) * pitch + (uint32_t)stage * 64);
    } else if (j < kPaW + kPwW) {
      const int i = min((j - kPaW) * NW + wave, kPw - 1);
      buffer_load_lds16(rwp, &sm.w[buf][i * 1024], voff_p,
                        (uint32_t)(n0 + 16 * i) * pitch + (uint32_t)stage * 64);
    } else {
      issue_scale(spair, t & 1, sb);
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

  // Fragments of two chunks (by the wave's own chunk order: 0 = first, 1 = second) and
  // decoded operands of two k-steps.
  const int xg0 = wave_m ? GS + 1 : 0;  // first whole activation group of this wave
  // lane's 16-byte piece of chunk 0 within a 32-row group (2 KiB); chunk 1's is 32 over
  const int fr0 = (r32 >> 4) * 1024 + (r32 & 15) * 64 + 16 * (h ^ chunk_swz(r32 & 15));
  const int wfrag = wave_n * FN * 2048;
  const int xfrag = xg0 * 2048;
  const int sfrag = GS * 2048;
  const int wsw = (kRowsSx + wave_n * FN * 32 + r32) * 16 + 2 * h;  // scale byte offsets
  const int xsw = (xg0 * 32 + r32) * 16 + 2 * h;
  const int ssw = (GS * 32 + r32) * 16 + 2 * h;
  u32x4 wraw[2][FN], xraw[2][FM], sraw;
  uint32_t wsr[2][FN], xsr[2][FM], ssr;
  half2_t wsc[FN], xsc[FM], ssc;
  half8_t wf[2][FN], xf[2][FM], sf[2];
  // read the fragments of chunk `c` (physical) of stage buffer `buf` as the wave's chunk
  // `par`, with the scales of the stage (pair buffer `sb`, stage `sub` of the pair); the
  // shared group only in its first chunk
  auto read_chunk = [&](int par, int buf, int c, int sb, int sub) {
    const int fr = fr0 ^ (32 * c);
    const uint8_t* wb = &sm.w[buf][wfrag + fr];
    const uint8_t* xb = &sm.x[buf][xfrag + fr];
    const uint8_t* scb = &sm.sc[sb][sub * 8 + c * 4];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[par][i] = *(const u32x4*)(wb + i * 2048);
      wsr[par][i] = *(const uint16_t*)(scb + wsw + i * 512);
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      xraw[par][f] = *(const u32x4*)(xb + f * 2048);
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

  // prologue: scales of pairs 0 and 1, codes of stages 0, 1 and 2
  issue_scale(0, 0, 0);
  issue_scale(0, 1, 0);
  issue_scale(npair > 1 ? 1 : 0, 0, 1);
  issue_scale(npair > 1 ? 1 : 0, 1, 1);
#pragma unroll
  for (int j = 0; j < kPaW + kPwW; ++j) issue(j, 0, 0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < kPaW + kPwW; ++j) issue(j, nk > 1 ? 1 : nk - 1, 1, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < kPaW + kPwW; ++j) issue(j, nk > 2 ? 2 : nk - 1, 2, 0, 0, 0);
  // stages 0 and 1 (stage 0 reads stage 1's first chunk ahead); stage 2's loads may
  // still be in flight: the wait at the end of stage 0 covers them
  wait_vmcnt<kPaW + kPwW>();
  __builtin_amdgcn_s_barrier();
  read_chunk(0, 0, wave_m, 0, 0);
  decode_step(0, 0, 0);

  int buf = 0;
  for (int t = 0; t < nk; ++t) {
    const int nbuf = (buf + 1) & 3;  // stage t + 1 (complete since the end of stage t - 2)
    const int lbuf = (buf + 3) & 3;  // stage t + 3 (its buffer held stage t - 1)
    const int lstage = t + 3 < nk ? t + 3 : nk - 1;
    const int pair = t >> 1;
    const int sb = pair % 3, sbn = ((t + 1) >> 1) % 3;        // pair buffers of t and t + 1
    const int spair = pair + 2 < npair ? pair + 2 : npair - 1;  // pair loaded in this stage
    const int sbl = (pair + 2) % 3;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int cur = st & 1;
      const int par = st >> 2, j = st & 3;
#pragma unroll
      for (int l = 0; l < kLoadsPerStep; ++l)
        if (st * kLoadsPerStep + l < kLoadsPerWave) issue(st * kLoadsPerStep + l, lstage, lbuf, t, spair, sbl);
      if (j == 0) {  // the wave's second chunk of this stage, or its first of the next
        if (par == 0) read_chunk(1, buf, wave_m ^ 1, sb, t & 1);
        else read_chunk(0, nbuf, wave_m, sbn, (t + 1) & 1);
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
          if (q < kLoadsPerStep && st * kLoadsPerStep + q < kLoadsPerWave)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global->LDS
          __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_GEMM_VALU_PER_MFMA, 0);  // VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<kLoadsPerWave>();
    __builtin_amdgcn_s_barrier();
    buf = nbuf;
  }

  // The two partial sums of the shared group: drain the last (unused) loads, then swap
  // them through LDS (the stage buffers are free now).
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
constexpr int kFuseElems = 16384;
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

  const __amdgpu_buffer_rsrc_t rxp = make_rsrc(p.a_packed, (uint32_t)p.M * pitch);
  const __amdgpu_buffer_rsrc_t rwp = make_rsrc(p.w_packed, (uint32_t)p.N * pitch);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.a_scales, (uint32_t)p.M * spitch);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.w_scales, (uint32_t)p.N * spitch);
  const uint32_t voff_p = r32 * pitch + h * 16;
  const uint32_t voff_s = r32 * spitch + h * 2;

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
  const uint32_t voff_sv = r32 * spitch;
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
              rwp, (int)voff_p, (int)((uint32_t)(n0 + 32 * i) * pitch + (uint32_t)c * 32), 0);
          if constexpr (!kVecScale)
            wsv[s][i][k] = __builtin_amdgcn_raw_buffer_load_b16(
                rws, (int)voff_s, (int)((uint32_t)(n0 + 32 * i) * spitch + (uint32_t)c * 4), 0);
        }
        if constexpr (!kFuse) {
#pragma unroll
          for (int g = 0; g < B; ++g) {
            xraw[s][k][g] = __builtin_amdgcn_raw_buffer_load_b128(
                rxp, (int)voff_p, (int)((uint32_t)(m0 + 32 * g) * pitch + (uint32_t)c * 32), 0);
            if constexpr (!kVecScale)
              xsv[s][g][k] = __builtin_amdgcn_raw_buffer_load_b16(
                  rxs, (int)voff_s, (int)((uint32_t)(m0 + 32 * g) * spitch + (uint32_t)c * 4), 0);
          }
        }
      }
    }
    if constexpr (kVecScale) {
      // a whole group: its 16 scale bytes lie inside the row; a partial last group takes
      // 4 bytes per chunk instead (same layout), so no load reaches past the row's end
      auto vec = [&](__amdgpu_buffer_rsrc_t r, int row0) -> u32x4 {
        const uint32_t base = (uint32_t)row0 * spitch + (uint32_t)c0 * 4;
        if (c0 + 4 <= nchunks) return (u32x4)__builtin_amdgcn_raw_buffer_load_b128(r, (int)voff_sv, (int)base, 0);
        u32x4 v{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c0 + k < nchunks) v[k] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff_sv, (int)(base + 4 * k), 0);
        return v;
      };
#pragma unroll
      for (int i = 0; i < A; ++i) wsv[s][i] = vec(rws, n0 + 32 * i);
      if constexpr (!kFuse) {
#pragma unroll
        for (int g = 0; g < B; ++g) xsv[s][g] = vec(rxs, m0 + 32 * g);
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

  // kFuse: quantize the M x K activations into LDS: half block hb (8 elements) per lane,
  // the pair (hb, hb ^ 1) being one block in lanes (2i, 2i + 1) of one wave.
  auto quantize_to_lds = [&]() {
    const QuantScale qsc = quant_scale(fq.gs, fq.den, fq.rden, fq.gs_dev);
    const int nhalves = (int)(p.M * p.K / 8);
    const u32x4* xv = (const u32x4*)fq.x;
    for (int hb = threadIdx.x; hb < nhalves; hb += 64 * NW) {
      float f[8];
      unpack_bf16x8(xv[hb], f);
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
      if (tn == 0 && fq.ws_packed != nullptr) {
        *(uint32_t*)(fq.ws_packed + 4 * (int64_t)hb) = word;
        if ((hb & 1) == 0) fq.ws_scales[hb >> 1] = (uint8_t)bs.code;
      }
    }
    __syncthreads();
  };

#pragma unroll
  for (int s = 0; s < DG; ++s)
    if (s < ngroups) load_group(s, s);
  // (after the first weight loads, so their latency overlaps the quantization)
  if constexpr (kFuse) quantize_to_lds();
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
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * q + e;
              float s = rb[v * 64 + lane];
#pragma unroll
              for (int w = 1; w < NW; ++w) s += rb[(w * 16 + v) * 64 + lane];
              b[e] = bf16_rne(apply_alpha<kExp>(s, alpha));
            }
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

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool aligned, int64_t cus) {
  constexpr int BM = kTileBM, BN = kTileBN, KC = kTileKC;
  constexpr int FBM = kFitBM, FBN = kFitBN;
  GemmPlan plan{};
  cus = cus > 0 ? cus : 256;
  // 32-bit buffer offsets (with one tile of rows past the end) for the 256x256, fit and
  // split-K kernels
  const bool fits32 = (M + FBM) * (K / 2) < ((int64_t)1 << 31) &&
                      (N + FBN) * (K / 2) < ((int64_t)1 << 31);
  const bool fits32_256 = (M + BM) * (K / 2) < ((int64_t)1 << 31) &&
                          (N + BN) * (K / 2) < ((int64_t)1 << 31);
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
  // activations once per 32 weight rows, which stops paying beyond that). Measured cost:
  // ~6000 cycles of launch and reduction plus, per pass over the chip, 360 / 740 / 1100
  // cycles per 128 elements of K for 32-row groups B = 1 / 2 / 4 per workgroup.
  const bool split_ok = aligned && K % 32 == 0 && fits32;
  const SplitShape sh = splitk_shape(M);
  const int64_t wsplit = ((N + 31) / 32) * ((M + 32 * sh.b - 1) / (32 * sh.b));
  const double csplit = 6000.0 + (double)passes(wsplit, cus) * ((double)K / 128.0) *
                                     (sh.b == 1 ? 360.0 : sh.b == 2 ? 740.0 : 1100.0);
  plan.kernel = fast ? NVFP4_GEMM_TILE256 : NVFP4_GEMM_GENERIC;
  plan.split = splitk_shape(M);
  if (fast || fit_ok) {
    double best = c256;
    if (fit_ok && cfit <= best) { plan.kernel = NVFP4_GEMM_FIT; best = cfit; }
    if (fast && c128 < best) { plan.kernel = NVFP4_GEMM_TILE128; best = c128; }
    if (fast && c128sq < best) { plan.kernel = NVFP4_GEMM_TILE128X128; best = c128sq; }
    if (fast && c12864 < best) { plan.kernel = NVFP4_GEMM_TILE128X64; best = c12864; }
    if (split_ok && M <= 512 && csplit < best) plan.kernel = NVFP4_GEMM_SPLITK;
  } else if (split_ok && M <= 512 && tfit * 4 <= cus) {
    // against the register-staged kernel (K % 128 != 0): few tiles only
    plan.kernel = NVFP4_GEMM_SPLITK;
  }
  return plan;
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream, const LaunchInfo& dev) {
  const bool aligned = ((uintptr_t)p.a_packed % 16 == 0) && ((uintptr_t)p.w_packed % 16 == 0) &&
                       ((uintptr_t)p.a_scales % 4 == 0) && ((uintptr_t)p.w_scales % 4 == 0);
  const GemmPlan plan = plan_gemm(p.M, p.N, p.K, aligned, dev.num_cus);
  switch (plan.kernel) {
    case NVFP4_GEMM_SPLITK:
      return launch_splitk(p, stream, plan.split);
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
    default:
      return launch_tile<kTileBM, kTileBN, kTileKC, NVFP4_GEMM_WM, NVFP4_GEMM_WN>(
          p, stream, plan.kernel == NVFP4_GEMM_TILE256);
  }
}

bool linear_fused(int64_t M, int64_t N, int64_t K, bool aligned, int64_t cus) {
  const GemmPlan g = plan_gemm(M, N, K, aligned, cus);
  // one 32-row activation group, and activations small enough to quantize in every
  // workgroup (and to sit in its LDS)
  return g.kernel == NVFP4_GEMM_SPLITK && M <= 32 && M * K <= kFuseElems;
}

hipError_t launch_linear_fused(const GemmProblem& p, const FusedQuant& fq, hipStream_t stream) {
  const int64_t wgs = (p.N + 31) / 32;
  if (p.M > 32 || p.M * p.K > kFuseElems || wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (p.K % 64 == 0)
    launch_splitk_kernel<1, 1, 4, 4, true, true>(dim3((unsigned)wgs), dim3(256), stream, p, fq);
  else
    launch_splitk_kernel<1, 1, 4, 4, true, false>(dim3((unsigned)wgs), dim3(256), stream, p, fq);
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
