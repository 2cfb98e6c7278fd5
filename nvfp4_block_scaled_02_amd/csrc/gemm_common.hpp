// Device helpers shared by the GEMM kernels (gemm.hip, gemm_w4a16.hip): operand decode
// of NVFP4 fragments, bf16 rounding of results and buffer resources.
#pragma once

#include "codec.hpp"
#include "kernels.hpp"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

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

// fp32 -> bf16, round to nearest even, on the bit pattern (the reference the hardware
// conversion below is checked against).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t b = f2u(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even bf16 by gfx950's packed conversion
// (v_cvt_pk_bf16_f32; a in the low half): one instruction where bf16_rne takes four
// integer operations per value. Equal to bf16_rne on every non-NaN binary32 pattern
// (nvfp4_selftest_bf16_exhaustive).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ u32x2 bf16x4_rne(float a, float b, float c, float d) {
  return u32x2{bf16x2_rne(a, b), bf16x2_rne(c, d)};
}

// Raw buffer resource over n bytes at p (gfx9-family descriptor word 3: 32-bit data
// format, no swizzle). The hardware range check compares only the per-lane offset
// (voffset plus the instruction's immediate) with n, dword by dword for multi-dword
// loads; the scalar offset (soffset) is added to the address but is NOT checked. A
// dword whose per-lane offset is >= n reads as zero and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// ---- row windows: how every range-checked operand load finds its row ---------------------
//
// A kernel that reads rows past the end of an operand (the ragged last tile of a GEMM)
// relies on the range check to turn those reads into zeros. Since only the per-lane
// offset is checked, the row of every load must be in that offset: each operand gets a
// resource based at the tile's first row row0 and covering rows [row0, rows), and a
// load's per-lane offset is (row - row0) * pitch plus whatever part of its position
// along K could leave the row; the scalar offset carries only a position along K that
// keeps the whole load inside its row. Then a row past the operand's end is out of range
// as a whole, and no in-range dword lies outside the operand.

// Bytes of the window of rows [row0, rows) (row0 < rows); the shape checks of the entry
// points keep (rows + one tile) * pitch below 2^31.
NVFP4_HD uint32_t window_bytes(int64_t row0, int64_t rows, uint32_t pitch) {
  return (uint32_t)((rows - row0) * (int64_t)pitch);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window_rsrc(const void* base, int64_t row0,
                                                              int64_t rows, uint32_t pitch) {
  return make_rsrc((const uint8_t*)base + row0 * (int64_t)pitch, window_bytes(row0, rows, pitch));
}

// Chunk swizzle of a 64-byte LDS row by its index r (0..15) within a 1 KiB piece of 16
// rows: the row's 16-byte chunk q is stored at slot q ^ chunk_swz(r). A lane (h, r) of an
// MFMA fragment reads chunk h or h + 2 of row r; with this swizzle the 16-byte reads of
// any 8 or 16 consecutive lanes fall in distinct LDS banks (32- or 64-bank view), and a
// direct-to-LDS load whose lane l fetches chunk (l % 4) ^ chunk_swz(l / 4) of row l / 4
// writes the piece in this order.
NVFP4_HD int chunk_swz(int r) { return ((r >> 1) + (r >> 3)) & 3; }

// Per-lane offset of a 16-row code piece load (16 rows x 64 bytes, four lanes per row):
// lane l reads row prow + l / 4 of the window, chunk (l % 4) ^ chunk_swz(l / 4) of the
// 64-byte segment that the scalar offset selects (a stage's position along K, inside
// the row).
NVFP4_HD uint32_t code_piece_voff(int lane, int prow, uint32_t pitch) {
  const int lr = lane >> 2;
  return (uint32_t)(prow + lr) * pitch + 16u * (uint32_t)((lane & 3) ^ chunk_swz(lr));
}

// Per-lane offset of a 64-row scale piece load (16 bytes of each of 64 rows): lane l reads
// row prow + l of the window at byte kbyte of the row. kbyte is part of the checked
// offset because the last piece of a row can extend past the row's end (a partial last
// group of stages): its dwords past the operand's end then read as zero.
NVFP4_HD uint32_t scale_piece_voff(int lane, int prow, uint32_t spitch, uint32_t kbyte) {
  return (uint32_t)(prow + lane) * spitch + kbyte;
}

// Per-lane offsets of the 16-row kernel's loads (gemm_gemv16_kernel) through a row window:
// lane (r, q) reads, of row r and 256-element group g of K (one 128-byte line of codes and
// 16 scale bytes per row), code bytes 32q + 16h .. + 15 (half h = 0, 1) and scale bytes
// 4q .. 4q + 3. The row is in the checked offset, and with K % 256 == 0 every load lies
// inside its row.
NVFP4_HD uint32_t gemv_code_voff(int r, int q, int h, int g, uint32_t pitch) {
  return (uint32_t)r * pitch + (uint32_t)g * 128u + 32u * (uint32_t)q + 16u * (uint32_t)h;
}
NVFP4_HD uint32_t gemv_scale_voff(int r, int q, int g, uint32_t spitch) {
  return (uint32_t)r * spitch + (uint32_t)g * 16u + 4u * (uint32_t)q;
}

// The W4A16 16-row kernel's bf16 activation loads: lane (r, q) reads 16 bytes k = 0..7 of
// its 128-byte quarter of group g (elements 64q + 8k .. + 7) of activation row r.
NVFP4_HD uint32_t gemv_x16_voff(int r, int q, int k, int g, uint32_t xpitch) {
  return (uint32_t)r * xpitch + (uint32_t)g * 512u + 128u * (uint32_t)q + 16u * (uint32_t)k;
}

// Swizzle of the W4A16 kernels' bf16 activation rows (128 bytes of a stage, eight 16-byte
// chunks): chunk c of row r (r = row within its 32-row group) sits at slot c ^ x_swz(r).
NVFP4_HD int x_swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// Per-lane offset of a W4A16 activation piece load (8 rows x 128 bytes, eight lanes per
// row): lane l reads row prow + l / 8 of the window, chunk (l % 8) ^ x_swz(row % 32) of
// the stage's 128-byte segment (selected by the scalar offset).
NVFP4_HD uint32_t x_piece_voff(int lane, int prow, uint32_t xpitch) {
  const int xr = lane >> 3;
  return (uint32_t)(prow + xr) * xpitch + 16u * (uint32_t)((lane & 7) ^ x_swz((prow + xr) & 31));
}

// The epilogue scale a_global * w_global (split as in split_alpha), from the launch
// arguments or, when the global scales are device-resident, from device memory (each
// value clamped as the quantizer clamps it, so a linear layer's two kernels agree).
__device__ __forceinline__ Alpha gemm_alpha(const GemmProblem& p) {
  if (p.a_gs_dev != nullptr)
    return split_alpha(clamp_global_scale(*p.a_gs_dev), clamp_global_scale(*p.w_gs_dev));
  return Alpha{p.alpha, p.alpha_exp};
}
// acc * a_global * w_global in fp32. With kExp = false (launches whose host scales
// multiply to a normal fp32, alpha.e == 0): one multiply and one rounding per element.
// With kExp = true (other host pairs, and device-resident scales, whose product the
// launch cannot see): the multiply by m, then 2^e by ldexp, which rounds a second time
// only where it takes a result below the normal range. The launchers pick the kernel
// instantiation, so the common epilogue keeps its single multiply (an ldexp per element
// costs 0.7% on the 4608 x 3072 x 3072 product).
template <bool kExp>
__device__ __forceinline__ float apply_alpha(float acc, const Alpha& al) {
  if constexpr (kExp) return __builtin_ldexpf(acc * al.m, al.e);
  else return acc * al.m;
}

// Epilogue shared by the GEMM kernels: lane holds, for weight group i and activation
// group g, output row m = m_base + 32g + (lane % 32) and columns
// n_base + 32i + 8q + 4(lane / 32) + {0..3} in acc[i][g][4q..4q+3]; each is multiplied
// by alpha (apply_alpha) in fp32, rounded to nearest even bf16 and stored (8 bytes per
// lane when the row pitch allows). Only column quads q in [q0, q1) are stored.
template <int FM, int FN, bool kExp = false>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[FN][FM], const GemmProblem& p,
                                           const Alpha alpha, int64_t m_base, int64_t n_base,
                                           int lane, int q0 = 0, int q1 = 4) {
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const bool n_vec = (p.N & 3) == 0;
#pragma unroll
  for (int g = 0; g < FM; ++g) {
    const int64_t m = m_base + g * 32 + r32;
    if (m >= p.M) continue;
    uint16_t* orow = p.out + m * p.N;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < q0 || q >= q1) continue;
        const int64_t n = n_base + i * 32 + 8 * q + 4 * h;
        const u32x2 w = bf16x4_rne(apply_alpha<kExp>(acc[i][g][4 * q], alpha),
                                   apply_alpha<kExp>(acc[i][g][4 * q + 1], alpha),
                                   apply_alpha<kExp>(acc[i][g][4 * q + 2], alpha),
                                   apply_alpha<kExp>(acc[i][g][4 * q + 3], alpha));
        if (n_vec && n + 3 < p.N) {
          *(u32x2*)&orow[n] = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) orow[n + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// The same stores through LDS: one 32-row group of the wave's blocks at a time is
// written, rounded, into the wave's own LDS area `blk` (32 rows of FN*32 bf16, rows
// kStoreRowPad(FN) elements apart) and read back as 16-byte row pieces, so each store
// instruction writes whole row segments (FN*64 bytes per row) instead of 16-byte pieces
// of 32 rows. The 16-byte row padding puts the 32 rows a lane group writes at once in
// different LDS banks. `blk` must not be used by other waves; LDS order within the wave
// makes the round trip safe without a barrier. The 16-byte row pieces are stored
// nontemporal (the kernel never reads its output back): measured on the 4608-row FLUX
// products 1-2% faster for the W4A4 and W4A16 kernels and 3-4% for the fp8 ones, while
// the same hint on store_tile's 8-byte pieces, which two waves fill half a cache line
// each, was 5% slower.
constexpr int kStoreRowPad(int fn) { return fn * 32 + 8; }

//
// kRowCol: instead of the scalar alpha, each output (m, n) is scaled by a_scales[m] *
// w_scales[n], read as fp32 arrays [M] and [N] (rowwise-scaled products); entries past M
// or N read as zero through range-checked buffer loads.
template <int FM, int FN, bool kRowCol = false, bool kExp = false>
__device__ __forceinline__ void store_tile_lds(const floatx16 (&acc)[FN][FM], const GemmProblem& p,
                                               const Alpha alpha, int64_t m_base, int64_t n_base,
                                               int lane, uint16_t* blk) {
  constexpr int W = FN * 32;            // columns of the wave's blocks
  constexpr int RS = kStoreRowPad(FN);  // row stride in the staging area
  constexpr int kPieces = 32 * W / 8;   // 16-byte pieces per 32-row group
  const int h = lane >> 5;
  const int r32 = lane & 31;
  const bool n_vec = (p.N & 7) == 0;  // 16-byte aligned row pieces
  float sx[FM];
  u32x4 sw[FN][4];
  if constexpr (kRowCol) {
    const __amdgpu_buffer_rsrc_t rsx = make_rsrc(p.a_scales, (uint32_t)(p.M * 4));
    const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.w_scales, (uint32_t)(p.N * 4));
#pragma unroll
    for (int g = 0; g < FM; ++g)
      sx[g] = u2f(__builtin_amdgcn_raw_buffer_load_b32(rsx, (int)((m_base + g * 32 + r32) * 4), 0, 0));
    // one dword per column (a 16-byte load straddling N could read as zero as a whole)
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sw[i][q][e] = __builtin_amdgcn_raw_buffer_load_b32(rsw, (int)((n_base + i * 32 + 8 * q + 4 * h + e) * 4), 0, 0);
  }
#pragma unroll
  for (int g = 0; g < FM; ++g) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (kRowCol) v[e] = acc[i][g][4 * q + e] * sx[g] * u2f(sw[i][q][e]);
          else v[e] = apply_alpha<kExp>(acc[i][g][4 * q + e], alpha);
        }
        *(u32x2*)&blk[r32 * RS + i * 32 + 8 * q + 4 * h] = bf16x4_rne(v[0], v[1], v[2], v[3]);
      }
    const int64_t m_row = m_base + g * 32;
#pragma unroll
    for (int it = 0; it < (kPieces + 63) / 64; ++it) {
      const int c = it * 64 + lane;
      if (c < kPieces) {
        const int r = c / (W / 8), col = (c % (W / 8)) * 8;
        const int64_t m = m_row + r, n = n_base + col;
        if (m < p.M) {
          const u32x4 v = *(const u32x4*)&blk[r * RS + col];
          if (n_vec && n + 7 < p.N) {
            __builtin_nontemporal_store(v, (u32x4*)&p.out[m * p.N + n]);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < p.N) p.out[m * p.N + n + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
}

typedef __attribute__((address_space(3))) void* lptr_t;

// Wait until at most n of this wave's vector memory operations are outstanding (n < 16;
// expcnt and lgkmcnt left free). Loads complete in issue order.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);
}

// Direct-to-LDS buffer loads: each lane reads 16 (4) bytes at voff + soff and writes
// them to lds_base + lane * 16 (4).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                  uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)lds_base, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                 uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)lds_base, 4, (int)voff, (int)soff, 0, 0);
}

#ifndef NVFP4_GEMM_XCD_GROUP
#define NVFP4_GEMM_XCD_GROUP 4
#endif
// Workgroup -> tile. Consecutive workgroups go to the 8 XCDs in turn and each XCD has its
// own L2, so workgroup b takes tile (b % 8) * (T / 8) + b / 8 of an order in which each
// XCD's share is contiguous; that order walks groups of G tile rows column by column, so
// an XCD's tiles share few activation and weight rows. (T % 8 != 0: plain order.)
__device__ __forceinline__ void tile_order(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcd = 8, G = NVFP4_GEMM_XCD_GROUP;
  const int T = tiles_m * tiles_n;
  if (G <= 0 || T % kXcd != 0) {
    tm = b / tiles_n;
    tn = b % tiles_n;
    return;
  }
  const int q = (b % kXcd) * (T / kXcd) + b / kXcd;
  const int per_group = G * tiles_n;
  const int gm0 = (q / per_group) * G;
  const int rows = min(tiles_m - gm0, G);
  const int r = q % per_group;
  tm = gm0 + r % rows;
  tn = r / rows;
}

}  // namespace
}  // namespace nvfp4
