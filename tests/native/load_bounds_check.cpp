// Host model of the range-checked operand loads of the GEMM kernels (gemm.hip, mxfp8.hip,
// gemm_w4a16.hip), driven by tests/test_load_bounds.py.
//
// Every such load reads through a buffer resource over a row window [row0, rows) of its
// operand (window_bytes), with a per-lane offset that the hardware range-checks dword by
// dword and a scalar offset that it does not check. For every tile, piece, lane, position
// along K and dword that a kernel can issue, this program evaluates the same offset
// helpers the kernels call (csrc/gemm_common.hpp) and checks:
//   (1) a dword whose per-lane offset is in range lies inside the operand
//       ([0, rows * pitch) bytes from its start): no access past the end of a buffer that
//       is exactly rows * pitch bytes long;
//   (2) a dword inside a real row (row < rows, byte position + 4 <= pitch) is in range and
//       reads that row's bytes at that position: no real data is zeroed or misplaced;
//   (3) a dword of a row past the end is out of range (reads as zero).
// Prints "<family> loads <n> violations <v>" per family and exits nonzero on a violation.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <functional>
#include <vector>

#include "gemm_common.hpp"

using namespace nvfp4;

namespace {

struct Stats {
  long long loads = 0, bad = 0;
};

// One load of `bytes` bytes (a multiple of 4, or 2 for a 16-bit load) at per-lane offset
// voff and scalar offset soff, through the window of rows [row0, rows) with `pitch` bytes
// per row. `row` and `pos` are the row (absolute) and byte position along the row that
// the kernel means to read.
void check_load(Stats& st, const char* fam, int64_t rows, uint32_t pitch, int64_t row0,
                uint32_t voff, uint32_t soff, int bytes, int64_t row, int64_t pos) {
  st.loads++;
  const uint32_t nrec = window_bytes(row0, rows, pitch);
  const int64_t size = rows * (int64_t)pitch;
  const int unit = bytes >= 4 ? 4 : bytes;
  for (int d = 0; d < bytes; d += unit) {
    const uint64_t v = (uint64_t)voff + (uint64_t)d;
    const bool in_range = v < nrec && v + unit <= nrec;
    const int64_t addr = row0 * (int64_t)pitch + (int64_t)v + (int64_t)soff;
    const bool real = row < rows && pos + d + unit <= (int64_t)pitch;
    bool ok = true;
    if (in_range && (addr < 0 || addr + unit > size)) ok = false;           // (1)
    if (real && (!in_range || addr != row * (int64_t)pitch + pos + d)) ok = false;  // (2)
    if (row >= rows && in_range) ok = false;                                // (3)
    if (!ok) {
      if (st.bad < 5)
        fprintf(stderr, "%s: rows=%lld pitch=%u row0=%lld row=%lld pos=%lld d=%d voff=%u soff=%u nrec=%u\n",
                fam, (long long)rows, pitch, (long long)row0, (long long)row, (long long)pos, d, voff,
                soff, nrec);
      st.bad++;
    }
  }
}

// Tiles of `tile` rows over `rows` rows (the window of each starts at its first row).
void for_tiles(int64_t rows, int tile, const std::function<void(int64_t)>& f) {
  for (int64_t r0 = 0; r0 < rows; r0 += tile) f(r0);
}

// Direct-to-LDS code pieces of 16 rows x 64 bytes at byte seg * 64 of the row: MXFP8's
// 256 x 256 tile (pitch K, scalar offset), or, with seg_in_voff, the W4A16 weight codes of
// a double stage (pitch K/2, the offset in the per-lane offset).
void code_pieces(Stats& st, const char* fam, int64_t rows, int64_t K, int tile, uint32_t pitch,
                 int nstage, bool seg_in_voff = false) {
  for_tiles(rows, tile, [&](int64_t r0) {
    for (int i = 0; i < tile / 16; ++i)
      for (int lane = 0; lane < 64; ++lane)
        for (int stage = 0; stage < nstage; ++stage) {
          const uint32_t so = (uint32_t)stage * 64;
          const uint32_t voff = code_piece_voff(lane, 16 * i, pitch) + (seg_in_voff ? so : 0);
          const int lr = lane >> 2;
          const int chunk = (lane & 3) ^ chunk_swz(lr);
          check_load(st, fam, rows, pitch, r0, voff, seg_in_voff ? 0 : so, 16, r0 + 16 * i + lr,
                     (int64_t)so + 16 * chunk);
        }
  });
  (void)K;
}

// Direct-to-LDS pieces of 8 rows x 128 bytes (eight lanes per row, chunk (l % 8) ^
// x_swz(row % 32)) at byte seg * 128 of the row: the W4A16 activations (pitch 2K, one stage
// per segment, scalar offset) and the double-stage MXFP8 / fp8r codes (pitch K, two
// stages per segment, scalar offset), or, with seg_in_voff, the double-stage NVFP4 codes
// (pitch K/2, the segment's offset in the per-lane offset: the last segment of an odd
// stage count reaches past the row's end).
void row128_pieces(Stats& st, const char* fam, int64_t rows, int tile, uint32_t pitch, int nseg,
                   bool seg_in_voff = false) {
  for_tiles(rows, tile, [&](int64_t r0) {
    for (int i = 0; i < tile / 8; ++i)
      for (int lane = 0; lane < 64; ++lane)
        for (int seg = 0; seg < nseg; ++seg) {
          const int xr = lane >> 3;
          const int chunk = (lane & 7) ^ x_swz((8 * i + xr) & 31);
          const uint32_t so = (uint32_t)seg * 128;
          check_load(st, fam, rows, pitch, r0, x_piece_voff(lane, 8 * i, pitch) + (seg_in_voff ? so : 0),
                     seg_in_voff ? 0 : so, 16, r0 + 8 * i + xr, (int64_t)so + 16 * chunk);
        }
  });
}

// Direct-to-LDS scale pieces: 64 rows x 16 bytes per piece at byte 16 * group of the row
// (a pair of NVFP4 stages, or 8 MXFP8 stages), `srows` rows per tile (rounded up to whole
// pieces, so the last piece may reach into the next tile).
void scale_pieces(Stats& st, const char* fam, int64_t rows, int tile, int srows, uint32_t spitch,
                  int ngroups) {
  for_tiles(rows, tile, [&](int64_t r0) {
    for (int i = 0; i < srows / 64; ++i)
      for (int lane = 0; lane < 64; ++lane)
        for (int g = 0; g < ngroups; ++g) {
          const uint32_t voff = scale_piece_voff(lane, 64 * i, spitch, (uint32_t)g * 16);
          check_load(st, fam, rows, spitch, r0, voff, 0, 16, r0 + 64 * i + lane, (int64_t)g * 16);
        }
  });
}

// Split-K kernel (NVFP4 W4A4): 32-row groups of a window of 32 * ngrp rows; lane (h, r)
// reads 16 code bytes at byte 32 c + 16 h and 2 scale bytes at 4 c + 2 h (or, with
// 16-byte scale loads, 16 bytes at 4 c0 for a whole group of four chunks, else 4 bytes per
// chunk).
void splitk(Stats& st, int64_t rows, int64_t K, int ngrp) {
  const uint32_t pitch = (uint32_t)(K / 2), spitch = (uint32_t)(K / 16);
  const int nchunks = (int)((K + 63) / 64);
  for_tiles(rows, 32 * ngrp, [&](int64_t r0) {
    for (int i = 0; i < ngrp; ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const int h = lane >> 5, r32 = lane & 31;
        const int64_t row = r0 + 32 * i + r32;
        for (int c = 0; c < nchunks; ++c) {
          const uint32_t cv = (uint32_t)(32 * i + r32) * pitch + (uint32_t)h * 16 + (uint32_t)c * 32;
          check_load(st, "splitk-codes", rows, pitch, r0, cv, 0, 16, row, (int64_t)c * 32 + 16 * h);
          const uint32_t sv = (uint32_t)(32 * i + r32) * spitch + (uint32_t)h * 2 + (uint32_t)c * 4;
          check_load(st, "splitk-scales16", rows, spitch, r0, sv, 0, 2, row, (int64_t)c * 4 + 2 * h);
        }
        if (K % 64 == 0)
          for (int c0 = 0; c0 < nchunks; c0 += 4) {
            const uint32_t v = (uint32_t)(32 * i + r32) * spitch + (uint32_t)c0 * 4;
            if (c0 + 4 <= nchunks) {
              check_load(st, "splitk-vecscales", rows, spitch, r0, v, 0, 16, row, (int64_t)c0 * 4);
            } else {
              for (int k = 0; c0 + k < nchunks; ++k)
                check_load(st, "splitk-vecscales", rows, spitch, r0, v + 4 * k, 0, 4, row,
                           (int64_t)(c0 + k) * 4);
            }
          }
      }
  });
}

// 16-row kernel (at most 32 activation rows): a window of rows [b R, rows) per workgroup b
// for the weights (lanes r < R load) and [0, M) for the activations (lane r loads rows r
// and 16 + r below M); lane (r, q) reads 16 code bytes at 128 g + 32 q + 16 h and 4 scale
// bytes at 16 g + 4 q of group g (K % 256 == 0).
void gemv16(Stats& st, int64_t rows, int64_t K, int R, bool weights) {
  const uint32_t pitch = (uint32_t)(K / 2), spitch = (uint32_t)(K / 16);
  const int ngt = (int)(K / 256);
  const int64_t step = weights ? R : rows;
  for (int64_t r0 = 0; r0 < rows; r0 += step)
    for (int slot = 0; slot < (weights ? 64 : 128); ++slot) {
      const int lane = slot & 63, r = (slot >> 6) * 16 + (lane & 15), q = lane >> 4;
      if (weights ? r >= R : r >= rows) continue;  // lanes that load nothing
      const int64_t row = r0 + r;
      for (int g = 0; g < ngt; ++g) {
        for (int h = 0; h < 2; ++h)
          check_load(st, "gemv16-codes", rows, pitch, r0, gemv_code_voff(r, q, h, g, pitch), 0, 16,
                     row, (int64_t)g * 128 + 32 * q + 16 * h);
        check_load(st, "gemv16-scales", rows, spitch, r0, gemv_scale_voff(r, q, g, spitch), 0, 4, row,
                   (int64_t)g * 16 + 4 * q);
      }
    }
}

// W4A16 16-row kernel's bf16 activation loads: window [0, M), rows r and 16 + r below M,
// 16 bytes k of the lane's 128-byte quarter of group g (K % 256 == 0).
void w4a16_gemv16_x(Stats& st, int64_t M, int64_t K) {
  const uint32_t xpitch = (uint32_t)(2 * K);
  for (int slot = 0; slot < 128; ++slot) {   // lanes of both activation blocks
    const int r = (slot >> 6) * 16 + (slot & 15), q = (slot & 63) >> 4;
    if (r >= M) continue;
    for (int g = 0; g < (int)(K / 256); ++g)
      for (int k = 0; k < 8; ++k)
        check_load(st, "w4a16-gemv16-x", M, xpitch, 0, gemv_x16_voff(r, q, k, g, xpitch), 0, 16, r,
                   (int64_t)g * 512 + 128 * q + 16 * k);
  }
}

// W4A16 256 x 256 and 288 x 192 kernels: activation pieces of 8 rows x 128 bytes (xpitch
// 2K, scalar offset stage * 128), weight groups of 32 rows x 32 bytes (stage * 32), scale
// pieces of 64 rows x 4 bytes (stage * 4); K % 64 == 0.
void w4a16_tiled(Stats& st, int64_t M, int64_t N, int64_t K, int BM, int BN) {
  const uint32_t xpitch = (uint32_t)(2 * K), pitch = (uint32_t)(K / 2), spitch = (uint32_t)(K / 16);
  const int nk = (int)(K / 64);
  for_tiles(M, BM, [&](int64_t m0) {
    for (int i = 0; i < BM / 8; ++i)
      for (int lane = 0; lane < 64; ++lane)
        for (int stage = 0; stage < nk; ++stage) {
          const int xr = lane >> 3;
          const int chunk = (lane & 7) ^ x_swz((8 * i + xr) & 31);
          check_load(st, "w4a16-x", M, xpitch, m0, x_piece_voff(lane, 8 * i, xpitch),
                     (uint32_t)stage * 128, 16, m0 + 8 * i + xr, (int64_t)stage * 128 + 16 * chunk);
        }
  });
  for_tiles(N, BN, [&](int64_t n0) {
    for (int stage = 0; stage < nk; ++stage)
      for (int lane = 0; lane < 64; ++lane) {
        const int h = lane >> 5, r32 = lane & 31;
        for (int i = 0; i < BN / 32; ++i)
          check_load(st, "w4a16-w", N, pitch, n0, (uint32_t)(32 * i + r32) * pitch + h * 16u,
                     (uint32_t)stage * 32, 16, n0 + 32 * i + r32, (int64_t)stage * 32 + 16 * h);
        for (int i = 0; i < (BN + 63) / 64; ++i)
          check_load(st, "w4a16-s", N, spitch, n0, (uint32_t)(64 * i + lane) * spitch,
                     (uint32_t)stage * 4, 4, n0 + 64 * i + lane, (int64_t)stage * 4);
      }
  });
}

// W4A16 split-K: window of 32 B activation rows at m0 and 32 weight rows at n0; lane
// (h, r) reads 4 x 16 bytes of activations at byte 128 c + 64 h (+16 j) of its row in
// group g, 16 code bytes at 32 c + 16 h and 2 scale bytes at 4 c + 2 h; K % 32 == 0.
void w4a16_splitk(Stats& st, int64_t M, int64_t N, int64_t K, int B) {
  const uint32_t xpitch = (uint32_t)(2 * K), pitch = (uint32_t)(K / 2), spitch = (uint32_t)(K / 16);
  const int nchunks = (int)((K + 63) / 64);
  for_tiles(M, 32 * B, [&](int64_t m0) {
    for (int lane = 0; lane < 64; ++lane) {
      const int h = lane >> 5, r32 = lane & 31;
      const uint32_t voff_x = r32 * xpitch + h * 64;
      for (int g = 0; g < B; ++g)
        for (int c = 0; c < nchunks; ++c)
          for (int j = 0; j < 4; ++j)
            check_load(st, "w4a16-splitk-x", M, xpitch, m0,
                       voff_x + (uint32_t)g * 32 * xpitch + (uint32_t)c * 128 + 16 * j, 0, 16,
                       m0 + 32 * g + r32, (int64_t)c * 128 + 64 * h + 16 * j);
    }
  });
  for_tiles(N, 32, [&](int64_t n0) {
    for (int lane = 0; lane < 64; ++lane) {
      const int h = lane >> 5, r32 = lane & 31;
      const uint32_t voff_w = r32 * pitch + h * 16, voff_s = r32 * spitch + h * 2;
      for (int c = 0; c < nchunks; ++c) {
        check_load(st, "w4a16-splitk-w", N, pitch, n0, voff_w + (uint32_t)c * 32, 0, 16, n0 + r32,
                   (int64_t)c * 32 + 16 * h);
        check_load(st, "w4a16-splitk-s", N, spitch, n0, voff_s + (uint32_t)c * 4, 0, 2, n0 + r32,
                   (int64_t)c * 4 + 2 * h);
      }
    }
  });
}

void report(const char* fam, const Stats& st, long long& bad) {
  printf("%s loads %lld violations %lld\n", fam, st.loads, st.bad);
  bad += st.bad;
}

}  // namespace

int main(int argc, char** argv) {
  // shapes: rows of the operand and K; ragged row counts around every tile size
  const int64_t rows_list[] = {1, 17, 31, 33, 64, 100, 129, 257, 289, 385, 777, 1000, 2305, 3073};
  long long bad = 0;
  {
    Stats st;
    const int64_t Ks[] = {128, 384, 640, 3072};
    for (int64_t R : rows_list)
      for (int64_t K : Ks)
        // every tile's double-stage loads (an odd stage count leaves half a segment)
        for (int tile : {288, 192, 256, 128, 64})
          row128_pieces(st, "nvfp4-codes-128", R, tile, (uint32_t)(K / 2), (int)(K / 128 + 1) / 2, true);
    report("nvfp4-code-pieces", st, bad);
  }
  {
    Stats st;
    const int64_t Ks[] = {128, 384, 640, 3072};
    for (int64_t R : rows_list)
      for (int64_t K : Ks)
        for (int tile : {288, 192, 256, 128, 64}) {
          const int nk = (int)(K / 128);
          scale_pieces(st, "nvfp4-scales", R, tile, (tile + 63) / 64 * 64, (uint32_t)(K / 16), (nk + 1) / 2);
        }
    report("nvfp4-scale-pieces", st, bad);
  }
  {
    Stats st;
    const int64_t Ks[] = {32, 96, 160, 384, 1056, 3072};
    for (int64_t R : rows_list)
      for (int64_t K : Ks)
        for (int ngrp : {1, 2, 4}) splitk(st, R, K, ngrp);
    report("splitk", st, bad);
  }
  {
    Stats st;
    const int64_t Ks[] = {256, 768, 3072};
    for (int64_t R : rows_list)
      for (int64_t K : Ks) {
        for (int wr : {4, 8, 12, 16}) gemv16(st, R, K, wr, true);
        if (R <= 32) gemv16(st, R, K, 16, false);
      }
    report("gemv16", st, bad);
  }
  {
    Stats st;
    for (int64_t M = 1; M <= 32; ++M)
      for (int64_t K : {256, 768, 3072}) w4a16_gemv16_x(st, M, K);
    report("w4a16-gemv16", st, bad);
  }
  {
    Stats st;
    const int64_t Ks[] = {128, 384, 640, 1152, 3072};
    for (int64_t R : rows_list)
      for (int64_t K : Ks)
        for (int tile : {288, 192, 256}) {
          const int nk = (int)(K / 64);
          code_pieces(st, "mxfp8-codes", R, K, tile, (uint32_t)K, nk);
          if (tile != 256) row128_pieces(st, "mxfp8-codes-128", R, tile, (uint32_t)K, nk / 2);
          scale_pieces(st, "mxfp8-scales", R, tile, (tile + 63) / 64 * 64, (uint32_t)(K / 32), (nk + 7) / 8);
        }
    report("mxfp8", st, bad);
  }
  {
    Stats st;
    const int64_t Ks[] = {64, 192, 320, 448, 3072};
    for (int64_t M : {1, 33, 289, 777, 1000})
      for (int64_t N : {17, 193, 385, 1000})
        for (int64_t K : Ks) {
          w4a16_tiled(st, M, N, K, 256, 256);
          w4a16_tiled(st, M, N, K, 288, 192);
          // the tiles along N: activations by stage, weight codes and scales by double
          // stage and quad, offsets in the per-lane offset
          for (int bm : {224, 128, 96, 64}) {
            const int nk = (int)(K / 64), nd = (nk + 1) / 2;
            row128_pieces(st, "w4a16-x", M, bm, (uint32_t)(2 * K), 2 * nd, true);
          }
          for (int bn : {256, 128}) {
            const int nk = (int)(K / 64), nd = (nk + 1) / 2;
            code_pieces(st, "w4a16-w", N, K, bn, (uint32_t)(K / 2), nd, true);
            scale_pieces(st, "w4a16-quad-s", N, bn, bn, (uint32_t)(K / 16), (nk + 3) / 4);
          }
        }
    report("w4a16-tiled", st, bad);
  }
  {
    Stats st;
    const int64_t Ks[] = {32, 96, 160, 3072};
    for (int64_t M : {1, 17, 33, 100, 257})
      for (int64_t N : {1, 17, 385})
        for (int64_t K : Ks)
          for (int B : {1, 2, 4}) w4a16_splitk(st, M, N, K, B);
    report("w4a16-splitk", st, bad);
  }
  (void)argc;
  (void)argv;
  printf("total violations %lld\n", bad);
  return bad ? 1 : 0;
}
