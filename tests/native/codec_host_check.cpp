// Host build of the quantizer's scalar codecs (nvfp4_block_scaled_02_amd/csrc/codec.hpp),
// driven by tests/test_codec_host.py, which compares every output with the CPU oracle.
//
//   division                 exhaustive: reciprocal + correction vs IEEE x / d for every
//                            bf16 significand of x in [1, 4) and binary32 significand of
//                            d in [1, 2); prints "mismatches <n>"
//   scale <in> <gs_hex> <out>   per float32 amax: block scale code (u8) and d (float32)
//   e2m1 <in> <out>          per float32 y: software E2M1 code of (x = y, y)
//   e4m3 <in> <out>          per float32 s >= 0: E4M3 code
//   e4m3dec <out>            float32 value of every code 0..126
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "codec.hpp"

using namespace nvfp4;

static std::vector<float> read_f32(const char* path) {
  FILE* f = fopen(path, "rb");
  if (!f) { perror(path); exit(2); }
  fseek(f, 0, SEEK_END);
  long n = ftell(f) / 4;
  fseek(f, 0, SEEK_SET);
  std::vector<float> v(n);
  if (fread(v.data(), 4, n, f) != (size_t)n) { perror("read"); exit(2); }
  fclose(f);
  return v;
}

static void write_bytes(const char* path, const void* p, size_t n) {
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, n, f) != n) { perror(path); exit(2); }
  fclose(f);
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  if (!strcmp(argv[1], "division")) {
    unsigned long long bad = 0;
    for (uint32_t dm = 0; dm < (1u << 23); ++dm) {
      const float d = u2f(0x3F800000u | dm);
      const float r = 1.0f / d;
      for (uint32_t xm = 0; xm < 256; ++xm) {
        const float x = u2f(((127u + (xm >> 7)) << 23) | ((xm & 127u) << 16));
        const float y = div_by_scale(x, d, r);
        const float q = x / d;
        if (f2u(y) != f2u(q)) {
          if (bad < 5) printf("x=%a d=%a y=%a q=%a\n", x, d, y, q);
          ++bad;
        }
        // negative x takes the same path with the sign flipped
        const float yn = div_by_scale(-x, d, r);
        if (f2u(yn) != (f2u(q) | 0x80000000u)) ++bad;
      }
    }
    // zeros keep their sign, for every divisor and for the d == 0 (r = 0) case
    for (uint32_t dm = 0; dm < (1u << 23); dm += 97) {
      const float d = u2f(0x3F800000u | dm);
      const float r = 1.0f / d;
      if (f2u(div_by_scale(0.0f, d, r)) != 0u) ++bad;
      if (f2u(div_by_scale(-0.0f, d, r)) != 0x80000000u) ++bad;
    }
    for (uint32_t xm = 0; xm < 65536; ++xm) {  // every finite bf16 pattern with d == 0
      if ((xm & 0x7F80u) == 0x7F80u) continue;  // inputs are finite by contract
      const float x = u2f(xm << 16);
      if (f2u(div_by_scale(x, 0.0f, 0.0f)) != (f2u(x) & 0x80000000u)) ++bad;
    }
    printf("mismatches %llu\n", bad);
    return 0;
  }
  if (!strcmp(argv[1], "scale") && argc == 5) {
    const std::vector<float> a = read_f32(argv[2]);
    const float gs = u2f((uint32_t)strtoul(argv[3], nullptr, 16));
    const float den = 6.0f * gs;
    std::vector<uint8_t> out(a.size() * 5);
    for (size_t i = 0; i < a.size(); ++i) {
      const BlockScale b = block_scale(a[i], den, gs);
      out[5 * i] = (uint8_t)b.code;
      memcpy(&out[5 * i + 1], &b.d, 4);
    }
    write_bytes(argv[4], out.data(), out.size());
    return 0;
  }
  if (!strcmp(argv[1], "e2m1") && argc == 4) {
    const std::vector<float> y = read_f32(argv[2]);
    std::vector<uint8_t> out(y.size());
    for (size_t i = 0; i < y.size(); ++i) out[i] = (uint8_t)e2m1_encode_sw(y[i], y[i]);
    write_bytes(argv[3], out.data(), out.size());
    return 0;
  }
  if (!strcmp(argv[1], "e4m3") && argc == 4) {
    const std::vector<float> s = read_f32(argv[2]);
    std::vector<uint8_t> out(s.size());
    for (size_t i = 0; i < s.size(); ++i) out[i] = (uint8_t)e4m3_encode_sat(s[i]);
    write_bytes(argv[3], out.data(), out.size());
    return 0;
  }
  if (!strcmp(argv[1], "e4m3dec") && argc == 3) {
    std::vector<float> v(127);
    for (uint32_t c = 0; c < 127; ++c) v[c] = e4m3_decode(c);
    write_bytes(argv[2], v.data(), v.size() * 4);
    return 0;
  }
  return 2;
}
