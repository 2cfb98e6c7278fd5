// W4A16 GEMM for gfx950: out[M, N] (bf16) = w_global * X[M, K] W_hat[N, K]^T with X
// bf16 (unquantized activations) and W_hat decoded from NVFP4 (E2M1 codes x per-16 E4M3
// scales).
//
// This is the pages' path for hardware without the fused FP4 kernel: the weights stay
// NVFP4 in memory and the activations are not quantized ("BFL (fp8r / nvfp4)", text
// under the Kernels table), so its results differ slightly from the W4A4 kernel. It also
// suits short activations, where the weights dominate the bytes.
//
// Arithmetic: a decoded weight q * s has at most 6 significant bits and is exact in bf16;
// a bf16 x times it is exact in fp32, so the bf16 MFMA forms exact products and
// accumulates in fp32. The weight decode goes through fp32 (gfx950 has no packed bf16
// multiply): the fp4 -> fp32 conversion gives q, one fp32 multiply by s, and a packed
// conversion to bf16 (exact). 16 VALU per 8 elements per lane; the activations need none.
//
// Structure: two forms, chosen by the number of output tiles.
//  * Long activations (more than a quarter of the compute units' worth of 256 x 256
//    tiles, K % 64 == 0, aligned operands): tiled kernels with the bf16 activations
//    staged in LDS and the weights 4-bit in LDS (288 x 192 and 256 x 256 tiles,
//    described below).
//  * Otherwise, split K inside the workgroup, as in the W4A4 short-activation kernel: a
// workgroup owns 32 weight rows x 32B activation rows; its 4 waves take interleaved
// 64-element chunks of K (wave w: chunks w, w+4, ...), load their fragments straight into
// registers D chunks ahead, and the four partial sums of each 32x32 block meet in LDS in
// a fixed order. K mapping as in the W4A4 kernels: lane half h feeds MFMA K-slots
// [8h, 8h+8) with chunk elements 32h + 8j .. 32h + 8j + 7 on k-step j, which for X is one
// 16-byte load of 8 consecutive bf16.
//
// Buffer resources start at the workgroup's first row, so offsets are tile-local (any M
// and N) and rows past M or N read as zero.
#include "gemm_common.hpp"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Eight E2M1 codes (element i in bits 4i..4i+3 of p) times the fp32 block scale s, as
// bf16 (exact). Every conversion result is consumed as a whole vector.
__device__ __forceinline__ bf16x8_t decode8_bf16(uint32_t p, float s) {
  const float2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
  const float2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1);
  const float2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2);
  const float2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3);
  const bf16x2_t b0 = __builtin_convertvector(q0 * s, bf16x2_t);
  const bf16x2_t b1 = __builtin_convertvector(q1 * s, bf16x2_t);
  const bf16x2_t b2 = __builtin_convertvector(q2 * s, bf16x2_t);
  const bf16x2_t b3 = __builtin_convertvector(q3 * s, bf16x2_t);
  return __builtin_bit_cast(bf16x8_t, u32x4{__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                                            __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3)});
}

// fp32 values of the two E4M3 scale codes in the low 16 bits of v (c0 in bits 0..7),
// by gfx950's fp8 conversion (exact: every E4M3 value is an fp32 value). Measured 6%
// faster on the tiled kernels than the branchy software decode.
__device__ __forceinline__ float2_t scales_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
}

template <int B, int D>
__global__ void __launch_bounds__(256) gemm_w4a16_kernel(W4A16Problem p) {
  constexpr int NW = 4;
  __shared__ float red[2][NW][16 * 64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int64_t tiles_m = (p.M + 32 * B - 1) / (32 * B);
  const int64_t tm = (int64_t)blockIdx.x % tiles_m;  // consecutive workgroups share weight rows
  const int64_t tn = (int64_t)blockIdx.x / tiles_m;
  const int64_t m0 = tm * 32 * B;
  const int64_t n0 = tn * 32;
  const uint32_t xpitch = (uint32_t)(p.K * 2);  // bytes per activation row
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);
  const int nchunks = (int)((p.K + 63) / 64);
  const int nq = (nchunks - wave + NW - 1) / NW;  // this wave's chunks

  auto clamp31 = [](int64_t n) { return (uint32_t)(n < 0x7FFFFFFF ? n : 0x7FFFFFFF); };
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x + m0 * p.K, clamp31((p.M - m0) * (int64_t)xpitch));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w_packed + n0 * pitch, clamp31((p.N - n0) * (int64_t)pitch));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.w_scales + n0 * spitch, clamp31((p.N - n0) * (int64_t)spitch));
  const uint32_t voff_x = r32 * xpitch + h * 64;
  const uint32_t voff_w = r32 * pitch + h * 16;
  const uint32_t voff_s = r32 * spitch + h * 2;

  floatx16 acc[B];
#pragma unroll
  for (int g = 0; g < B; ++g)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[g][v] = 0.0f;

  u32x4 wraw[D], xraw[D][B][4];
  uint32_t wsr[D];
  auto load = [&](int d, int q) {
    const uint32_t c = (uint32_t)(wave + NW * q);
    wraw[d] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)voff_w, (int)(c * 32), 0);
    wsr[d] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)voff_s, (int)(c * 4), 0);
#pragma unroll
    for (int g = 0; g < B; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xraw[d][g][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rx, (int)(voff_x + 16 * j), (int)((uint32_t)g * 32 * xpitch + c * 128), 0);
  };
  auto compute = [&](int d, int q) {
    // upper lane half of a 32-element last chunk: no elements (its loads read the next
    // row or zeros), so both its weights and its activations are forced to zero
    const bool dead = h == 1 && (int64_t)(wave + NW * q) * 64 + 32 >= p.K;
    const uint32_t sw = dead ? 0u : wsr[d];
    const float2_t sf = scales_to_f32(sw);
    const float s_lo = sf[0], s_hi = sf[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t wf = decode8_bf16(wraw[d][j], j < 2 ? s_lo : s_hi);
#pragma unroll
      for (int g = 0; g < B; ++g) {
        const u32x4 xv = dead ? u32x4{0u, 0u, 0u, 0u} : xraw[d][g][j];
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, __builtin_bit_cast(bf16x8_t, xv), acc[g], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nq) load(d, d);
  for (int q = 0; q < nq; q += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (q + d < nq) {
        compute(d, q + d);
        if (q + d + D < nq) load(d, q + d + D);
      }
    }
  }

  // Partial sums: block by block, every wave writes its part, the owner wave (block
  // number % 4) adds the four in wave order and stores.
  const bool n_vec = (p.N & 3) == 0;
#pragma unroll
  for (int g = 0; g < B; ++g) {
    float* rb = red[g & 1][0];
#pragma unroll
    for (int v = 0; v < 16; ++v) rb[(wave * 16 + v) * 64 + lane] = acc[g][v];
    __syncthreads();
    if (wave == g % NW) {
      const int64_t m = m0 + g * 32 + r32;
      if (m < p.M) {
        uint16_t* orow = p.out + m * p.N;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int64_t n = n0 + 8 * qd + 4 * h;
          uint32_t b[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * qd + e;
            float s = rb[(0 * 16 + v) * 64 + lane];
            s += rb[(1 * 16 + v) * 64 + lane];
            s += rb[(2 * 16 + v) * 64 + lane];
            s += rb[(3 * 16 + v) * 64 + lane];
            b[e] = bf16_rne(s * p.alpha);
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

// ---- tiled form for long activations -------------------------------------------------
//
// 256 x 256 output tiles, 2 x 2 waves of 128 x 128 (4 x 4 blocks of 32 x 32), the bf16
// MFMA with the decoded weights as its A operand. A stage is 64 elements of K:
//  * activations: 256 rows x 128 bytes (bf16). A direct-to-LDS load fills 8 rows x 128
//    bytes (8 lanes per row, 1 KiB). In LDS each row's 16-byte chunk c sits at slot
//    c ^ x_swz(r) (r = row within its 32-row group), so the fragment reads (lane (h, r)
//    reads chunk 4h + j on k-step j) hit distinct banks;
//  * weights: 256 rows x 32 bytes of codes (per 32-row group 64 slots of 16 bytes in
//    MFMA lane order, loaded as 32 rows x 32 bytes) and 256 rows x 4 scale bytes.
// Three stage buffers (3 x 41 KiB); stage t+2's loads are issued during stage t; at the
// end of stage t each wave waits for the loads it issued before stage t and the
// workgroup meets at a barrier, so stage t+1 is complete when it starts. A stage reads
// its fragments k-step by k-step, one k-step ahead of its MFMAs.
__device__ __forceinline__ int x_swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

template <int BM, int BN>
struct alignas(16) W4A16Smem {
  uint8_t x[3][BM * 128];
  uint8_t w[3][BN * 32];
  uint8_t ws[3][BN * 4];
};

// Requires K % 64 == 0, 16-byte aligned x, codes and out, 4-byte aligned scales, and
// (M + 256) * K * 2 and (N + 256) * K / 2 below 2^31 (32-bit buffer offsets).
template <int BM, int BN>
__global__ void __launch_bounds__(256) gemm_w4a16_tile_kernel(W4A16Problem p) {
  constexpr int NW = 4, WM = 2, WN = 2;
  __shared__ W4A16Smem<BM, BN> sm;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  constexpr int kPx = BM / 8, kPw = BN / 32, kPs = BN / 64;  // loads per stage
  static_assert(kPx % NW == 0 && kPw % NW == 0 && kPs % NW == 0, "loads divide among waves");
  constexpr int kPxW = kPx / NW, kPwW = kPw / NW, kPsW = kPs / NW;
  constexpr int kLoads = kPxW + kPwW + kPsW;
  static_assert(kLoads < 16, "one stage of loads fits the vmcnt immediate");

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
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int nk = (int)(p.K / 64);
  const uint32_t xpitch = (uint32_t)(p.K * 2), pitch = (uint32_t)(p.K >> 1), spitch = (uint32_t)(p.K >> 4);

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)p.M * xpitch);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w_packed, (uint32_t)p.N * pitch);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.w_scales, (uint32_t)p.N * spitch);
  const int xr = lane >> 3;  // row (within 8) of an activation load
  const uint32_t voff_w = r32 * pitch + h * 16;
  const uint32_t voff_s = lane * spitch;

  // load j of this wave (lists: activation pieces, weight pieces, scale pieces)
  auto issue = [&](int j, int stage, int buf) {
    if (j < kPxW) {
      const int i = j * NW + wave;  // rows 8i .. 8i+7 of the tile
      const int row = 8 * i + xr;
      const uint32_t voff = xr * xpitch + 16 * ((lane & 7) ^ x_swz(row & 31));
      buffer_load_lds16(rx, &sm.x[buf][i * 1024], voff, (uint32_t)(m0 + 8 * i) * xpitch + (uint32_t)stage * 128);
    } else if (j < kPxW + kPwW) {
      const int i = (j - kPxW) * NW + wave;  // weight group i
      buffer_load_lds16(rw, &sm.w[buf][i * 1024], voff_w, (uint32_t)(n0 + 32 * i) * pitch + (uint32_t)stage * 32);
    } else {
      const int i = (j - kPxW - kPwW) * NW + wave;  // weight rows 64i .. 64i+63
      buffer_load_lds4(rs, &sm.ws[buf][i * 256], voff_s, (uint32_t)(n0 + 64 * i) * spitch + (uint32_t)stage * 4);
    }
  };

  floatx16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  const int xs0 = 16 * ((4 * h) ^ x_swz(r32));  // k-step j: slot offset xs0 ^ (16 j)
  u32x4 wraw[FN];
  float wsc_lo[FN], wsc_hi[FN];
  bf16x8_t wf[2][FN], xf[2][FM];
  auto read_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[i] = *(const u32x4*)&sm.w[buf][(wave_n * FN + i) * 1024 + lane * 16];
      const uint32_t sw = *(const uint16_t*)&sm.ws[buf][(wave_n * FN * 32 + i * 32 + r32) * 4 + 2 * h];
      const float2_t sf = scales_to_f32(sw);
      wsc_lo[i] = sf[0];
      wsc_hi[i] = sf[1];
    }
  };
  auto read_x = [&](int slot, int buf, int j) {
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      const u32x4 v = *(const u32x4*)&sm.x[buf][(wave_m * FM + g) * 4096 + r32 * 128 + (xs0 ^ (16 * j))];
      xf[slot][g] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  auto decode_w = [&](int slot, int j) {
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[slot][i] = decode8_bf16(wraw[i][j], j < 2 ? wsc_lo[i] : wsc_hi[i]);
  };

  // prologue: stages 0 and 1
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, nk > 1 ? 1 : 0, 1);
  wait_vmcnt<kLoads>();
  __builtin_amdgcn_s_barrier();

  int buf = 0;
  for (int t = 0; t < nk; ++t) {
    const int lbuf = buf == 0 ? 2 : buf - 1;  // (t + 2) % 3
    const int lstage = t + 2 < nk ? t + 2 : nk - 1;
    read_w(buf);
    read_x(0, buf, 0);
    decode_w(0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cur = j & 1;
      if (j < 3) {
        read_x(cur ^ 1, buf, j + 1);
        decode_w(cur ^ 1, j + 1);
      }
#pragma unroll
      for (int l = 0; l < (kLoads + 3) / 4; ++l)
        if (j * ((kLoads + 3) / 4) + l < kLoads) issue(j * ((kLoads + 3) / 4) + l, lstage, lbuf);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
    }
    wait_vmcnt<kLoads>();
    __builtin_amdgcn_s_barrier();
    buf = buf == 2 ? 0 : buf + 1;
  }

  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  GemmProblem q{};
  q.out = p.out;
  q.M = p.M;
  q.N = p.N;
  q.K = p.K;
  q.alpha = p.alpha;
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  store_tile_lds<FM, FN>(acc, q, Alpha{q.alpha, 0}, (int64_t)m0 + wave_m * FM * 32,
                         (int64_t)n0 + wave_n * FN * 32, lane,
                         (uint16_t*)&sm.x[0][0] + wave * 32 * kStoreRowPad(FN));
}


// ---- 288 x 192 tiles: every FLUX product in whole multiples of 256 tiles -------------
//
// The W4A4 fit tile's shape (4608 = 16 x 288; 3072, 9216, 12288 are multiples of 192)
// on the tiled form's loads and stage pipeline. 2 x 2 waves: wave (m, n) owns weight
// groups 3n .. 3n+2 and activation groups 0-3 (m = 0) or 5-8 (m = 1); the middle group 4
// is split by weight group, wave (0, n) taking groups 3n and 3n+1, wave (1, n) group
// 3n+2. Both read the middle activation fragment straight from LDS (activations need no
// decode here), and wave (1, n) also issues a second middle MFMA whose result it drops,
// so every wave issues 14 MFMAs per k-step with no branch in the loop. Loads per stage:
// 36 activation pieces (8 rows x 128 bytes), 6 weight pieces, 3 scale pieces, spread
// over the waves (slots past the last piece repeat it: identical data to the same LDS
// bytes). Three stage buffers (3 x 42.75 KiB).
template <int BM, int BN>
struct alignas(16) W4A16FitSmem {
  uint8_t x[3][BM * 128];
  uint8_t w[3][BN * 32];
  uint8_t ws[3][BN * 4];
};

// Requires K % 64 == 0, 16-byte aligned x, codes and out, 4-byte aligned scales, and
// (M + BM) * K * 2 and (N + BN) * K / 2 below 2^31 (32-bit buffer offsets).
template <int BM, int BN>
__global__ void __launch_bounds__(256) gemm_w4a16_fit_kernel(W4A16Problem p) {
  constexpr int NW = 4, WN = 2;
  __shared__ W4A16FitSmem<BM, BN> sm;
  constexpr int GX = BM / 32, GW = BN / 32;
  static_assert(GX * 32 == BM && GW * 32 == BN && GX % 2 == 1 && GW % WN == 0, "tile shape");
  constexpr int GS = GX / 2;      // the middle activation group
  constexpr int FM = GX / 2;      // own activation groups per wave
  constexpr int FN = GW / WN;     // weight groups per wave
  static_assert(FN == 3, "middle split: two weight groups for wave row 0, one for row 1");
  constexpr int kPx = BM / 8, kPw = GW, kPs = (BN + 63) / 64;  // pieces per stage
  constexpr int kPxW = (kPx + NW - 1) / NW, kPwW = (kPw + NW - 1) / NW, kPsW = (kPs + NW - 1) / NW;
  constexpr int kLoads = kPxW + kPwW + kPsW;
  static_assert(kLoads < 16, "one stage of loads fits the vmcnt immediate");

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
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int nk = (int)(p.K / 64);
  const uint32_t xpitch = (uint32_t)(p.K * 2), pitch = (uint32_t)(p.K >> 1), spitch = (uint32_t)(p.K >> 4);

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)p.M * xpitch);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w_packed, (uint32_t)p.N * pitch);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.w_scales, (uint32_t)p.N * spitch);
  const int xr = lane >> 3;  // row (within 8) of an activation load
  const uint32_t voff_w = r32 * pitch + h * 16;
  const uint32_t voff_s = lane * spitch;

  // load j of this wave (lists: activation pieces, weight pieces, scale pieces)
  auto issue = [&](int j, int stage, int buf) {
    if (j < kPxW) {
      const int i = min(j * NW + wave, kPx - 1);  // rows 8i .. 8i+7 of the tile
      const int row = 8 * i + xr;
      const uint32_t voff = xr * xpitch + 16 * ((lane & 7) ^ x_swz(row & 31));
      buffer_load_lds16(rx, &sm.x[buf][i * 1024], voff, (uint32_t)(m0 + 8 * i) * xpitch + (uint32_t)stage * 128);
    } else if (j < kPxW + kPwW) {
      const int i = min((j - kPxW) * NW + wave, kPw - 1);  // weight group i
      buffer_load_lds16(rw, &sm.w[buf][i * 1024], voff_w, (uint32_t)(n0 + 32 * i) * pitch + (uint32_t)stage * 32);
    } else {
      const int i = min((j - kPxW - kPwW) * NW + wave, kPs - 1);  // weight rows 64i .. 64i+63
      buffer_load_lds4(rs, &sm.ws[buf][i * 256], voff_s, (uint32_t)(n0 + 64 * i) * spitch + (uint32_t)stage * 4);
    }
  };

  floatx16 acc[FN][FM], accm[2];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int g = 0; g < FM; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) accm[k][v] = 0.0f;

  const int xg0 = wave_m == 0 ? 0 : GS + 1;  // first own activation group
  const int xs0 = 16 * ((4 * h) ^ x_swz(r32));  // k-step j: slot offset xs0 ^ (16 j)
  u32x4 wraw[FN];
  float wsc_lo[FN], wsc_hi[FN];
  bf16x8_t wf[2][FN], xf[2][FM + 1];  // xf[.][FM]: the middle group
  auto read_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[i] = *(const u32x4*)&sm.w[buf][(wave_n * FN + i) * 1024 + lane * 16];
      const uint32_t sw = *(const uint16_t*)&sm.ws[buf][(wave_n * FN * 32 + i * 32 + r32) * 4 + 2 * h];
      const float2_t sf = scales_to_f32(sw);
      wsc_lo[i] = sf[0];
      wsc_hi[i] = sf[1];
    }
  };
  auto read_x = [&](int slot, int buf, int j) {
#pragma unroll
    for (int g = 0; g <= FM; ++g) {
      const int grp = g < FM ? xg0 + g : GS;
      const u32x4 v = *(const u32x4*)&sm.x[buf][grp * 4096 + r32 * 128 + (xs0 ^ (16 * j))];
      xf[slot][g] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  auto decode_w = [&](int slot, int j) {
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[slot][i] = decode8_bf16(wraw[i][j], j < 2 ? wsc_lo[i] : wsc_hi[i]);
  };

  // prologue: stages 0 and 1
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, 0, 0);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, nk > 1 ? 1 : 0, 1);
  wait_vmcnt<kLoads>();
  __builtin_amdgcn_s_barrier();

  int buf = 0;
  for (int t = 0; t < nk; ++t) {
    const int lbuf = buf == 0 ? 2 : buf - 1;  // (t + 2) % 3
    const int lstage = t + 2 < nk ? t + 2 : nk - 1;
    read_w(buf);
    read_x(0, buf, 0);
    decode_w(0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cur = j & 1;
      if (j < 3) {
        read_x(cur ^ 1, buf, j + 1);
        decode_w(cur ^ 1, j + 1);
      }
#pragma unroll
      for (int l = 0; l < (kLoads + 3) / 4; ++l)
        if (j * ((kLoads + 3) / 4) + l < kLoads) issue(j * ((kLoads + 3) / 4) + l, lstage, lbuf);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
      // middle group: row 0 takes weight groups 0 and 1 of the wave, row 1 group 2 (and
      // a dropped product with group 1)
      const bf16x8_t m0w = wave_m == 0 ? wf[cur][0] : wf[cur][2];
      accm[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m0w, xf[cur][FM], accm[0], 0, 0, 0);
      accm[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][1], xf[cur][FM], accm[1], 0, 0, 0);
    }
    wait_vmcnt<kLoads>();
    __builtin_amdgcn_s_barrier();
    buf = buf == 2 ? 0 : buf + 1;
  }

  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  GemmProblem q{};
  q.out = p.out;
  q.M = p.M;
  q.N = p.N;
  q.K = p.K;
  q.alpha = p.alpha;
  uint16_t* stage_area = (uint16_t*)&sm.x[0][0] + wave * 32 * kStoreRowPad(FN);
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  const int64_t n_base = (int64_t)n0 + wave_n * FN * 32;
  store_tile_lds<FM, FN>(acc, q, Alpha{q.alpha, 0}, (int64_t)m0 + xg0 * 32, n_base, lane,
                         stage_area);
  if (wave_m == 0)
    store_tile_lds<1, 2>(*(const floatx16(*)[2][1])&accm, q, Alpha{q.alpha, 0},
                         (int64_t)m0 + GS * 32, n_base, lane, stage_area);
  else
    store_tile_lds<1, 1>(*(const floatx16(*)[1][1])&accm[0], q, Alpha{q.alpha, 0},
                         (int64_t)m0 + GS * 32, n_base + 64, lane, stage_area);
}

}  // namespace

hipError_t launch_gemm_w4a16(const W4A16Problem& p, hipStream_t stream, const LaunchInfo& dev) {
  // long activations: a tiled kernel when its tiles cover at least a quarter of the
  // compute units (as the W4A4 planner); 288 x 192 unless 256 x 256 tiles need fewer
  // passes (measured: 4608 x 3072 x 3072 88.7 us vs 90.4 us, x 12288 x 3072 352.5 vs 365.7)
  const int64_t cus = dev.num_cus > 0 ? dev.num_cus : 256;
  const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  const int64_t tfit = ((p.M + 287) / 288) * ((p.N + 191) / 192);
  const bool fits32 = (p.M + 288) * p.K * 2 < ((int64_t)1 << 31) && (p.N + 256) * (p.K / 2) < ((int64_t)1 << 31);
  const bool aligned = (uintptr_t)p.x % 16 == 0 && (uintptr_t)p.w_packed % 16 == 0 &&
                       (uintptr_t)p.w_scales % 4 == 0;
  if (p.K % 64 == 0 && fits32 && aligned && tiles * 4 > cus) {
    if (tiles > 0x7FFFFFFF || tfit > 0x7FFFFFFF) return hipErrorInvalidValue;
    // passes over the compute units weighted by MFMAs per wave and k-step (14 vs 16)
    const int64_t pf = (tfit + cus - 1) / cus, p256 = (tiles + cus - 1) / cus;
    if (pf * 14 <= p256 * 16)
      hipLaunchKernelGGL((gemm_w4a16_fit_kernel<288, 192>), dim3((unsigned)tfit), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_w4a16_tile_kernel<256, 256>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  // workgroup shape: 32 weight rows x 32B activation rows, B the smallest of 1, 2, 4 that
  // covers min(M, 128) rows
  const int B = p.M <= 32 ? 1 : (p.M <= 64 ? 2 : 4);
  const int64_t wgs = ((p.N + 31) / 32) * ((p.M + 32 * B - 1) / (32 * B));
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs), block(256);
  if (B == 1) hipLaunchKernelGGL((gemm_w4a16_kernel<1, 6>), grid, block, 0, stream, p);
  else if (B == 2) hipLaunchKernelGGL((gemm_w4a16_kernel<2, 4>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((gemm_w4a16_kernel<4, 2>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
