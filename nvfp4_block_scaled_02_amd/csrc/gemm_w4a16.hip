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
  // Every load's per-lane offset holds its row within the window and its whole position
  // along K (the upper lane half of a 32-element last chunk reads past its row, past the
  // operand's end for the last row), so the range check covers both.
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
    wraw[d] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(voff_w + c * 32), 0, 0);
    wsr[d] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(voff_s + c * 4), 0, 0);
#pragma unroll
    for (int g = 0; g < B; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xraw[d][g][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rx, (int)(voff_x + (uint32_t)g * 32 * xpitch + c * 128 + 16 * j), 0, 0);
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
          float sv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * qd + e;
            float s = rb[(0 * 16 + v) * 64 + lane];
            s += rb[(1 * 16 + v) * 64 + lane];
            s += rb[(2 * 16 + v) * 64 + lane];
            s += rb[(3 * 16 + v) * 64 + lane];
            sv[e] = s * p.alpha;
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

// ---- at most 16 activation rows: weight rows spread over the whole chip ------------------
//
// The layout of the NVFP4 16-row kernel (gemm.hip) with bf16 activations: a workgroup owns
// R <= 16 weight rows (gemv16_rows: 12 at N = 3072, 256 workgroups), its NW waves take the
// 256-element groups of K in turn, and a 16 x 16 x 32 bf16 MFMA block holds the R weight
// rows against up to 16 activation rows. Lane (r, q) loads 32 code bytes and 4 scale
// bytes of weight row r (elements 64q .. 64q + 63 of the group) and the same 64 elements
// of activation row r (128 bytes); word j of code half h, decoded to bf16 exactly, meets
// activation bytes 16(4h + j) .. + 15 (the same elements 64q + 32h + 8j .. + 7) in MFMA
// 4h + j. Lanes past the R weight rows or the M activation rows load nothing. The NW
// partial sums meet in LDS in wave order.
//
// Requires M <= 16, K % 256 == 0, 16-byte aligned x, packed weights and output, 4-byte
// aligned scales, and operands below 2^31 bytes.
template <int NW, int DG, int B>
__global__ void __launch_bounds__(64 * NW) gemm_w4a16_gemv16_kernel(W4A16Problem p, int R) {
  typedef float floatx4 __attribute__((ext_vector_type(4)));
  __shared__ floatx4 red[NW][B][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const uint32_t pitch = (uint32_t)(p.K >> 1);
  const uint32_t spitch = (uint32_t)(p.K >> 4);
  const uint32_t xpitch = (uint32_t)(p.K * 2);
  const int ngt = (int)(p.K / 256);
  const int ng = (ngt - wave + NW - 1) / NW;  // this wave's groups: wave, wave + NW, ...
  const bool wlive = r < R;
  const __amdgpu_buffer_rsrc_t rwp = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rws = window_rsrc(p.w_scales, n0, p.N, spitch);
  const __amdgpu_buffer_rsrc_t rx = window_rsrc(p.x, 0, p.M, xpitch);

  u32x4 wc[DG][2], xc[DG][B][8];
  uint32_t wsv[DG];
  auto load = [&](int s, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wc[s][h] = u32x4{0u, 0u, 0u, 0u};
      if (wlive)
        wc[s][h] = __builtin_amdgcn_raw_buffer_load_b128(rwp, (int)gemv_code_voff(r, q, h, g, pitch), 0, 0);
    }
    wsv[s] = 0u;
    if (wlive) wsv[s] = __builtin_amdgcn_raw_buffer_load_b32(rws, (int)gemv_scale_voff(r, q, g, spitch), 0, 0);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xc[s][b][k] = u32x4{0u, 0u, 0u, 0u};
        if (16 * b + r < p.M)
          xc[s][b][k] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)gemv_x16_voff(16 * b + r, q, k, g, xpitch), 0, 0);
      }
  };
  floatx4 acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // word j of half h: block 4q + 2h + j / 2, byte 2h + j / 2 of the lane's scale word
      const float2_t sf = scales_to_f32(wsv[s] >> (16 * h));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t wf = decode8_bf16(wc[s][h][j], j < 2 ? sf[0] : sf[1]);
#pragma unroll
        for (int b = 0; b < B; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, __builtin_bit_cast(bf16x8_t, xc[s][b][4 * h + j]),
                                                           acc[b], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int s = 0; s < DG; ++s)
    if (s < ng) load(s, wave + NW * s);
  for (int i = 0; i < ng; i += DG) {
#pragma unroll
    for (int s = 0; s < DG; ++s) {
      if (i + s < ng) {
        compute(s);
        if (i + s + DG < ng) load(s, wave + NW * (i + s + DG));
      }
    }
  }

  // lane (r, q) holds output rows 16b + r, columns n0 + 4q + {0..3} in acc[b]; wave 0 adds
  // the NW parts in wave order, scales, rounds and stores them
#pragma unroll
  for (int b = 0; b < B; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  if (wave != 0) return;
  const int64_t n = n0 + 4 * q;
  if (4 * q >= R || n >= p.N) return;
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
    for (int e = 0; e < 4; ++e) sv[e] = tot[e] * p.alpha;
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

  // row windows [m0, M) and [n0, N) (see window_rsrc): rows past M or N read as zero
  const __amdgpu_buffer_rsrc_t rx = window_rsrc(p.x, m0, p.M, xpitch);
  const __amdgpu_buffer_rsrc_t rw = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rs = window_rsrc(p.w_scales, n0, p.N, spitch);

  // load j of this wave (lists: activation pieces, weight pieces, scale pieces)
  auto issue = [&](int j, int stage, int buf) {
    if (j < kPxW) {
      const int i = j * NW + wave;  // rows 8i .. 8i+7 of the tile
      buffer_load_lds16(rx, &sm.x[buf][i * 1024], x_piece_voff(lane, 8 * i, xpitch), (uint32_t)stage * 128);
    } else if (j < kPxW + kPwW) {
      const int i = (j - kPxW) * NW + wave;  // weight group i: lane (h, r) row 32i + r, half h
      buffer_load_lds16(rw, &sm.w[buf][i * 1024], (uint32_t)(32 * i + r32) * pitch + h * 16u,
                        (uint32_t)stage * 32);
    } else {
      const int i = (j - kPxW - kPwW) * NW + wave;  // weight rows 64i .. 64i+63
      buffer_load_lds4(rs, &sm.ws[buf][i * 256], (uint32_t)(64 * i + lane) * spitch, (uint32_t)stage * 4);
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

  // row windows [m0, M) and [n0, N) (see window_rsrc): rows past M or N read as zero
  const __amdgpu_buffer_rsrc_t rx = window_rsrc(p.x, m0, p.M, xpitch);
  const __amdgpu_buffer_rsrc_t rw = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rs = window_rsrc(p.w_scales, n0, p.N, spitch);

  // load j of this wave (lists: activation pieces, weight pieces, scale pieces)
  auto issue = [&](int j, int stage, int buf) {
    if (j < kPxW) {
      const int i = min(j * NW + wave, kPx - 1);  // rows 8i .. 8i+7 of the tile
      buffer_load_lds16(rx, &sm.x[buf][i * 1024], x_piece_voff(lane, 8 * i, xpitch), (uint32_t)stage * 128);
    } else if (j < kPxW + kPwW) {
      const int i = min((j - kPxW) * NW + wave, kPw - 1);  // weight group i
      buffer_load_lds16(rw, &sm.w[buf][i * 1024], (uint32_t)(32 * i + r32) * pitch + h * 16u,
                        (uint32_t)stage * 32);
    } else {
      const int i = min((j - kPxW - kPwW) * NW + wave, kPs - 1);  // weight rows 64i .. 64i+63
      buffer_load_lds4(rs, &sm.ws[buf][i * 256], (uint32_t)(64 * i + lane) * spitch, (uint32_t)stage * 4);
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

// ---- tiles with the waves side by side along N (224 x 256 and smaller) -------------------
//
// Each wave owns BN/4 weight rows and all BM activation rows: at 224 x 256, two weight
// groups and seven activation groups, 14 MFMAs per k-step as in the 288 x 192 tile, but
// every weight group is decoded by one wave only (the 2 x 2 layouts decode each weight
// group in both wave rows), and a stage moves 13% fewer bytes per product. 4608 rows make
// 21 tile rows (the last one 128 rows); every FLUX width is a multiple of 256. The smaller
// forms (128 x 256, 96 x 256, 128 x 128, 64 x 128) serve short and medium activations.
//
// Loads. Direct-to-LDS loads cost by the cache lines they touch, so every load reads whole
// row segments: activations 8 rows x 128 bytes (a stage of one row: a whole line), weight
// codes 16 rows x 64 bytes (two stages of one row), the weights' scales 64 rows x 16 bytes
// (four stages: 4 bytes per row and stage). Loads go by double stage (128 elements of K):
// two double-stage buffers for the codes (each holding its two stages' activations and
// the weight rows' 64 bytes, 16-byte chunks swizzled by chunk_swz), two quad buffers for
// the scales. A double stage's byte offset rides in the per-lane offset, so when the
// stage count is odd the unused half of the last double stage is range-checked (zero past
// the operand's end).
//
// Pipeline over double stages d (stages 2d, 2d+1, buffers d & 1): each k-step reads and
// decodes the next k-step's fragments under its MFMAs; stage 2d's last k-step reads stage
// 2d+1's weights and first activation fragments (same buffer); in stage 2d+1's last
// k-step the wave first waits for all its loads (double stage d+1's, issued a double
// stage earlier) with its LDS reads landed and meets the workgroup at the double stage's
// one barrier, then reads double stage d+1's first fragments and issues double stage
// d+2's loads into buffer d & 1, whose reads all ended before the barrier.
template <int BM, int BN>
struct alignas(16) W4A16WideSmem {
  uint8_t x[2][2][BM * 128];  // [double stage buffer][stage of the pair][rows]
  uint8_t w[2][BN * 64];
  uint8_t ws[2][BN * 16];
};

#ifndef NVFP4_W4A16_VALU_PER_MFMA
#define NVFP4_W4A16_VALU_PER_MFMA 4
#endif

// Requires K % 64 == 0, 16-byte aligned x, codes and out, 4-byte aligned scales, and
// (M + BM) * K * 2 and (N + BN) * K / 2 below 2^31 (32-bit buffer offsets). The grid is
// the tile count rounded up to a multiple of 8; workgroups past the last tile exit.
template <int BM, int BN>
__global__ void __launch_bounds__(256) gemm_w4a16_wide_kernel(W4A16Problem p) {
  constexpr int NW = 4;
  __shared__ W4A16WideSmem<BM, BN> sm;
  constexpr int FM = BM / 32, FN = BN / NW / 32;
  constexpr int kPx = 2 * (BM / 8), kPw = BN / 16, kPs = BN / 64;  // pieces per double stage / quad
  static_assert(FM * 32 == BM && FN * 32 * NW == BN && BN % 64 == 0, "tile shape");
  static_assert(kPx % NW == 0 && kPw % NW == 0 && kPs <= NW, "loads divide among waves");
  constexpr int kPxW = kPx / NW, kPwW = kPw / NW;
  constexpr int kCode = kPxW + kPwW;              // code loads per wave and double stage
  constexpr int kLoads = kCode + 1;               // with a quad's scale piece
  static_assert(2 * kLoads < 64, "two double stages of loads fit the vmcnt counter");
  constexpr int kMfma = FN * FM;
  // A double stage's loads in two parts: the first kPartA after the barrier of the double
  // stage two before it (spread over the MFMAs of that last k-step), the rest over the
  // next stage (the first stage of the double stage before it). Tiles with few MFMAs per
  // k-step (64 x 128) have short stages and issue all of them after the barrier: their
  // second part would have too little lead (measured, 256 x 3072 x 12288: 63.3 us split,
  // 59.8 all after the barrier).
  constexpr int kPartA = kMfma >= 4 ? (kMfma < kCode ? kMfma : kCode) : kLoads;
  constexpr int kPerA = (kPartA + kMfma - 1) / kMfma;
  constexpr int kPerSlotB = kPartA >= kLoads ? 0 : (kLoads - kPartA + 4 * kMfma - 1) / (4 * kMfma);
  static_assert(kPartA < 16, "the prologue's wait fits the vmcnt immediate");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  // tile_order on the tile count rounded up to a multiple of 8 (the XCD count); the
  // slots past the last tile own nothing
  const int T = tiles_m * tiles_n;
  const int Tp = (T + 7) & ~7;
  const int b = (int)blockIdx.x;
  const int q = (b % 8) * (Tp / 8) + b / 8;
  if (q >= T) return;
  int tile_m, tile_n;
  {
    constexpr int G = NVFP4_GEMM_XCD_GROUP > 0 ? NVFP4_GEMM_XCD_GROUP : 1;
    const int per_group = G * tiles_n;
    const int gm0 = (q / per_group) * G;
    const int rows = min(tiles_m - gm0, G);
    const int r = q % per_group;
    tile_m = gm0 + r % rows;
    tile_n = r / rows;
  }
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int nk = (int)(p.K / 64);   // stages
  const int nd = (nk + 1) >> 1;     // double stages
  const int nquad = (nk + 3) >> 2;  // scale quads (two double stages)
  const uint32_t xpitch = (uint32_t)(p.K * 2), pitch = (uint32_t)(p.K >> 1), spitch = (uint32_t)(p.K >> 4);

  // row windows [m0, M) and [n0, N) (see window_rsrc): rows past M or N read as zero
  const __amdgpu_buffer_rsrc_t rx = window_rsrc(p.x, m0, p.M, xpitch);
  const __amdgpu_buffer_rsrc_t rw = window_rsrc(p.w_packed, n0, p.N, pitch);
  const __amdgpu_buffer_rsrc_t rs = window_rsrc(p.w_scales, n0, p.N, spitch);

  // Load j of this wave for double stage ds into buffer buf: activation pieces (stage
  // half, then rows 8i .. 8i+7), weight pieces (rows 16i .. 16i+15), then, when ds starts
  // a quad (ds even), that quad's scale piece (waves past the last piece repeat it: the
  // same bytes to the same LDS place). Loads for a double stage past the last reload the
  // last into a buffer no stage reads.
  auto issue = [&](int j, int dsn, int buf) {
    const int ds = dsn < nd ? dsn : nd - 1;
    if (j < kPxW) {
      const int i = j * NW + wave;
      const int half = i / (BM / 8), pi = i % (BM / 8);
      buffer_load_lds16(rx, &sm.x[buf][half][pi * 1024],
                        x_piece_voff(lane, 8 * pi, xpitch) + (uint32_t)(2 * ds + half) * 128, 0);
    } else if (j < kCode) {
      const int i = (j - kPxW) * NW + wave;
      buffer_load_lds16(rw, &sm.w[buf][i * 1024], code_piece_voff(lane, 16 * i, pitch) + (uint32_t)ds * 64, 0);
    } else {
      const int i = min(wave, kPs - 1);  // weight rows 64i .. 64i+63
      const int quad = min(dsn >> 1, nquad - 1);
      buffer_load_lds16(rs, &sm.ws[(dsn >> 1) & 1][i * 1024],
                        scale_piece_voff(lane, 64 * i, spitch, (uint32_t)quad * 16), 0);
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
  // lane's 16-byte weight chunk (stage half hs: chunk 2 hs + h) within a group of 32 rows
  const int wrow = (r32 >> 4) * 1024 + (r32 & 15) * 64;
  const int wsw = chunk_swz(r32 & 15);
  // weight codes and scale bytes of two stages (by stage parity), fragments of two k-steps
  u32x4 wraw[2][FN];
  uint32_t wsb[2][FN];
  bf16x8_t wf[2][FN], xf[2][FM];
  // stage st: double stage buffer buf, stage half hs = st & 1, scale quad st >> 2
  auto read_w = [&](int ws, int buf, int st) {
    const int hs = st & 1;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      wraw[ws][i] = *(const u32x4*)&sm.w[buf][(wave * FN + i) * 2048 + wrow + 16 * ((2 * hs + h) ^ wsw)];
      wsb[ws][i] = *(const uint16_t*)&sm.ws[(st >> 2) & 1][(wave * FN * 32 + i * 32 + r32) * 16 + 4 * (st & 3) + 2 * h];
    }
  };
  auto read_x = [&](int slot, int buf, int hs, int j) {
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      const u32x4 v = *(const u32x4*)&sm.x[buf][hs][g * 4096 + r32 * 128 + (xs0 ^ (16 * j))];
      xf[slot][g] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  // k-step j of the stage whose weights are in wraw[ws]: lane half h's 8 elements of each
  // weight group sit in 16-element block 2h + j / 2 of the stage's four (scale byte j / 2)
  auto decode_w = [&](int slot, int ws, int j) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const float2_t sf = scales_to_f32(wsb[ws][i]);
      wf[slot][i] = decode8_bf16(wraw[ws][i][j], j < 2 ? sf[0] : sf[1]);
    }
  };

  // prologue: double stages 0 and 1 (quad 0's scales with 0); wait for 0, read stage 0's
  // weights and first activation fragments
#pragma unroll
  for (int j = 0; j < kLoads; ++j) issue(j, 0, 0);
  constexpr int kPartA1 = kPartA < kCode ? kPartA : kCode;  // double stage 1 has no quad
#pragma unroll
  for (int j = 0; j < kPartA1; ++j) issue(j, 1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70 | kPartA1);
  __builtin_amdgcn_s_barrier();
  read_w(0, 0, 0);
  read_x(0, 0, 0, 0);
  decode_w(0, 0, 0);

  // stage half hs (a constant) of double stage d in buffer bb = d & 1 (a constant); ws = hs
  auto stage = [&](int d, const int bb, const int hs) {
    const int st = 2 * d + hs;
    // loads of this stage: part A of double stage d+2 (odd stage, after the barrier) or
    // part B of double stage d+1 (even stage); a double stage of even index starts a quad
    const int lds_ = hs == 1 ? d + 2 : d + 1;
    const int lbuf = hs == 1 ? bb : bb ^ 1;
    const int nl = (hs == 1 ? bb == 0 : bb == 1) ? kLoads : kCode;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cur = j & 1;
      const bool loads = hs == 0 || j == 3;
      if (j < 3) {
        read_x(cur ^ 1, bb, hs, j + 1);
        decode_w(cur ^ 1, hs, j + 1);
      } else if (hs == 0) {
        read_w(1, bb, st + 1);  // stage 2d+1, same buffer
        read_x(0, bb, 1, 0);
        decode_w(0, 1, 0);
      } else {
        // vmcnt(0) and lgkmcnt(0): double stage d+1 loaded, this wave's reads of bb done
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        read_w(0, bb ^ 1, st + 1);  // double stage d+1's first stage
        read_x(0, bb ^ 1, 0, 0);
        decode_w(0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cur][i], xf[cur][g], acc[i][g], 0, 0, 0);
      // order: one MFMA, then an LDS read, global->LDS loads and VALU work; after the
      // barrier the decode starts once the reads have had four MFMAs to land
#pragma unroll
      for (int qq = 0; qq < kMfma; ++qq) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (qq < FM + 2 * FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        if (loads && hs == 1) {
#pragma unroll
          for (int l = 0; l < kPerA; ++l) {
            const int idx = qq * kPerA + l;
            if (idx < kPartA && idx < nl) {
              issue(idx, lds_, lbuf);
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
          }
        } else if (loads && kPerSlotB > 0) {
#pragma unroll
          for (int l = 0; l < kPerSlotB; ++l) {
            const int idx = kPartA + (j * kMfma + qq) * kPerSlotB + l;
            if (idx < nl) {
              issue(idx, lds_, lbuf);
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
          }
        }
        if (j < 3 || qq >= 4) __builtin_amdgcn_sched_group_barrier(0x002, NVFP4_W4A16_VALU_PER_MFMA, 0);
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

  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  GemmProblem gq{};
  gq.out = p.out;
  gq.M = p.M;
  gq.N = p.N;
  gq.K = p.K;
  gq.alpha = p.alpha;
  static_assert(NW * 32 * kStoreRowPad(FN) * 2 <= sizeof(sm.x), "store staging fits");
  store_tile_lds<FM, FN>(acc, gq, Alpha{gq.alpha, 0}, (int64_t)m0, (int64_t)n0 + wave * FN * 32,
                         lane, (uint16_t*)&sm.x[0][0][0] + wave * 32 * kStoreRowPad(FN));
}

}  // namespace

namespace {

struct WideShape {
  W4A16Kernel kind;
  int bm, bn;
};
// the tiles with their waves along N, largest first
constexpr WideShape kWide[] = {{W4A16Kernel::kWide, 224, 256},
                               {W4A16Kernel::kWide128x256, 128, 256},
                               {W4A16Kernel::kWide96x256, 96, 256},
                               {W4A16Kernel::kWide128x128, 128, 128},
                               {W4A16Kernel::kWide64x128, 64, 128}};

// Cost of one stage (64 elements of K) of one tile, in 64-byte row segments loaded per
// compute unit: the tiled kernels' loads cost about 2.1 cycles per segment whatever the
// bytes used (measured over these tile shapes at one tile per compute unit), and a tile
// whose MFMAs take longer than its loads pays those instead (14 or 16 MFMAs of 32 cycles
// per wave and k-step for the largest tiles). Activation loads touch 16 segments per
// 8 rows; weight codes 32 per 32 rows; scales 64 per 64 rows, every stage (288 x 192,
// 256 x 256) or every fourth stage (the tiles along N).
double tile_stage_cost(int bm, int bn, bool quad_scales) {
  const double segs = 2.0 * bm + bn + (quad_scales ? bn / 4.0 : (double)bn);
  const double mfma = (double)(bm / 32) * (bn / 32) / 4.0 * 4.0 * 32.0 / 2.1;  // per wave
  return segs > mfma ? segs : mfma;
}

}  // namespace

W4A16Kernel plan_gemm_w4a16(int64_t M, int64_t N, int64_t K, int64_t num_cus, bool aligned) {
  // Activations of at most 64 rows: split-K (it reads the weights once and fills the chip
  // with 32-row workgroups). Longer ones: the tiled kernel with the fewest passes over the
  // compute units times its stage cost.
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const bool fits32 = fits_i31(M + 288, 2 * K) && fits_i31(N + 256, K / 2);
  // at most 16 rows (K % 256 == 0): the weights' read spread over the whole chip, up to
  // three passes of 16-row workgroups (its 186 VGPRs hold one 512-thread workgroup per
  // compute unit; measured: 1 x 12288 x 3072 10.2 us against split-K's 11.9, 8 x 18432 x
  // 3072 20.3 against 18.9); 17 to 32 rows (two activation blocks, a two-deep ring) in
  // one pass only
  const int64_t g16 = (N + 15) / 16;
  if (aligned && K % 256 == 0 && (M <= 16 ? g16 <= 3 * cus : (M <= 32 && g16 <= cus)) &&
      fits_i31(M + 32, 2 * K) && fits_i31(N + 16, K / 2))
    return W4A16Kernel::kGemv16;
  if (K % 64 != 0 || !fits32 || !aligned || M <= 64) return W4A16Kernel::kSplitK;
  auto cost = [&](int bm, int bn, bool quad) {
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    return (double)((tiles + cus - 1) / cus) * tile_stage_cost(bm, bn, quad);
  };
  W4A16Kernel best = W4A16Kernel::kFit;
  double cbest = cost(288, 192, false);
  const double c256 = cost(256, 256, false);
  if (c256 < cbest) { best = W4A16Kernel::kTile256; cbest = c256; }
  for (const WideShape& w : kWide) {
    const double c = cost(w.bm, w.bn, true);
    if (c <= cbest) { best = w.kind; cbest = c; }
  }
  return best;
}

hipError_t launch_gemm_w4a16(const W4A16Problem& p, hipStream_t stream, const LaunchInfo& dev) {
  const bool aligned = (uintptr_t)p.x % 16 == 0 && (uintptr_t)p.w_packed % 16 == 0 &&
                       (uintptr_t)p.w_scales % 4 == 0 && (uintptr_t)p.out % 16 == 0;
  const W4A16Kernel kind = plan_gemm_w4a16(p.M, p.N, p.K, dev.num_cus, aligned);
  auto tiles_of = [&](int bm, int bn, bool round8) -> int64_t {
    const int64_t t = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    return round8 ? (t + 7) & ~(int64_t)7 : t;
  };
  switch (kind) {
    case W4A16Kernel::kWide:
    case W4A16Kernel::kWide128x256:
    case W4A16Kernel::kWide96x256:
    case W4A16Kernel::kWide128x128:
    case W4A16Kernel::kWide64x128: {
      int bm = 0, bn = 0;
      for (const WideShape& w : kWide)
        if (w.kind == kind) { bm = w.bm; bn = w.bn; }
      const int64_t g = tiles_of(bm, bn, true);
      if (g > 0x7FFFFFF8) return hipErrorInvalidValue;
      const dim3 gd((unsigned)g), bd(256);
      if (kind == W4A16Kernel::kWide) hipLaunchKernelGGL((gemm_w4a16_wide_kernel<224, 256>), gd, bd, 0, stream, p);
      else if (kind == W4A16Kernel::kWide128x256) hipLaunchKernelGGL((gemm_w4a16_wide_kernel<128, 256>), gd, bd, 0, stream, p);
      else if (kind == W4A16Kernel::kWide96x256) hipLaunchKernelGGL((gemm_w4a16_wide_kernel<96, 256>), gd, bd, 0, stream, p);
      else if (kind == W4A16Kernel::kWide128x128) hipLaunchKernelGGL((gemm_w4a16_wide_kernel<128, 128>), gd, bd, 0, stream, p);
      else hipLaunchKernelGGL((gemm_w4a16_wide_kernel<64, 128>), gd, bd, 0, stream, p);
      return hipGetLastError();
    }
    case W4A16Kernel::kFit: {
      const int64_t t = tiles_of(288, 192, false);
      if (t > 0x7FFFFFFF) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_w4a16_fit_kernel<288, 192>), dim3((unsigned)t), dim3(256), 0, stream, p);
      return hipGetLastError();
    }
    case W4A16Kernel::kTile256: {
      const int64_t t = tiles_of(256, 256, false);
      if (t > 0x7FFFFFFF) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_w4a16_tile_kernel<256, 256>), dim3((unsigned)t), dim3(256), 0, stream, p);
      return hipGetLastError();
    }
    case W4A16Kernel::kGemv16: {
      const int R = gemv16_rows(p.N, dev.num_cus > 0 ? dev.num_cus : 256);
      const int64_t wgs = (p.N + R - 1) / R;
      if (wgs > 0x7FFFFFFF || p.M > 32 || p.K % 256 != 0) return hipErrorInvalidValue;
      // eight waves once K has eight groups (more loads in flight per compute unit); one or
      // two 16-row activation blocks
      const bool wide = p.K / 256 >= 8;
      const dim3 gd((unsigned)wgs);
      if (p.M <= 16) {
        if (wide) hipLaunchKernelGGL((gemm_w4a16_gemv16_kernel<8, 4, 1>), gd, dim3(512), 0, stream, p, R);
        else hipLaunchKernelGGL((gemm_w4a16_gemv16_kernel<4, 4, 1>), gd, dim3(256), 0, stream, p, R);
      } else {
        if (wide) hipLaunchKernelGGL((gemm_w4a16_gemv16_kernel<8, 2, 2>), gd, dim3(512), 0, stream, p, R);
        else hipLaunchKernelGGL((gemm_w4a16_gemv16_kernel<4, 2, 2>), gd, dim3(256), 0, stream, p, R);
      }
      return hipGetLastError();
    }
    case W4A16Kernel::kSplitK:
      break;
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
