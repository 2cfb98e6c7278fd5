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
        const float yu = div_by_scale_unclamped(x, d, r);
        const float q = x / d;
        if (f2u(y) != f2u(q) || f2u(yu) != f2u(q)) {
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
  if (!strcmp(argv[1], "extremes")) {
    // Random significand pairs at the extreme exponents the validated global-scale range
    // allows: d = s * gs in [2^-99, 2^99] (s in [2^-9, 448], gs in [2^-90, 2^90]) with
    // quotients x / d in [2^-3, 2^4) (the range that decides a code), for both quotient
    // forms; and the block-scale quotient amax / den with den = 6 * gs at the range ends.
    unsigned long long bad = 0, n = 0;
    uint64_t st = 0x9E3779B97F4A7C15ull;
    auto rnd = [&]() { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)(st >> 11); };
    const int dexp[] = {-99, -98, -97, -90, 88, 95, 98};
    for (int de : dexp) {
      for (int it = 0; it < 4000000; ++it) {
        const float d = u2f(((uint32_t)(de + 127) << 23) | (rnd() & 0x7FFFFFu));
        const int qe = (int)(rnd() % 7) - 3;
        const float x = u2f(((uint32_t)(de + qe + 127) << 23) | ((rnd() & 0x7Fu) << 16));
        const float r = 1.0f / d;
        const float q = x / d;
        ++n;
        // unclamped: exact everywhere; clamped: exact below 8, saturating (>= 6) above
        const float yc = div_by_scale(x, d, r);
        const bool ok_c = q < 8.0f ? f2u(yc) == f2u(q) : yc >= 6.0f;
        if (!ok_c || f2u(div_by_scale_unclamped(x, d, r)) != f2u(q)) {
          if (bad < 5) printf("x=%a d=%a\n", x, d);
          ++bad;
        }
      }
    }
    const float gss[] = {0x1p-90f, 0x1.8p-90f, 0x1p90f, 0x1.fffffep89f};
    for (float gs : gss) {
      const float den = 6.0f * gs, rden = 1.0f / den;
      for (int it = 0; it < 4000000; ++it) {
        const int qe = (int)(rnd() % 21) - 11;  // s_raw in [2^-11, 2^10)
        const int ae = (int)((f2u(den) >> 23) & 0xFF) - 127 + qe;
        const float amax = u2f(((uint32_t)(ae + 127) << 23) | ((rnd() & 0x7Fu) << 16));
        const BlockScale b = block_scale(amax, den, rden, gs);
        const uint32_t want = e4m3_encode_sat(amax / den);
        ++n;
        if (b.code != want) {
          if (bad < 5) printf("amax=%a den=%a\n", amax, den);
          ++bad;
        }
      }
    }
    printf("checked %llu mismatches %llu\n", n, bad);
    return 0;
  }
  if (!strcmp(argv[1], "scale") && argc == 5) {
    const std::vector<float> a = read_f32(argv[2]);
    const float gs = u2f((uint32_t)strtoul(argv[3], nullptr, 16));
    const float den = 6.0f * gs;
    const float rden = 1.0f / den;
    std::vector<uint8_t> out(a.size() * 5);
    for (size_t i = 0; i < a.size(); ++i) {
      const BlockScale b = block_scale(a[i], den, rden, gs);
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
