/*
 * libnvfp4 self-test entry points: they run, on the GPU, exactly the device functions
 * the quantize and GEMM kernels use (codec.hpp and the GEMM decode), so tests can check
 * them against the CPU oracle exhaustively or on chosen inputs. They are not part of
 * the compute path; all follow the conventions and status codes of nvfp4.h (device
 * pointers, asynchronous on `stream`, validation before any HIP call).
 *
 * The rounding rules checked here are those of the NVFP4 format: E2M1 elements with one
 * E4M3 scale per 16-element block ("BFL (fp8r / nvfp4)", nvfp4 item; zubnet.ai page,
 * paragraph 1), with the rounding conventions stated in nvfp4.h.
 */
#ifndef NVFP4_SELFTEST_H_
#define NVFP4_SELFTEST_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* For each binary32 y[i]: hw_codes[i] = the gfx950 conversion instruction's E2M1 code
 * (scale 1.0), sw_codes[i] = the software encoder's code (sign of y, nearest magnitude,
 * ties to even, saturating at 6). n >= 0 elements; outputs are one code per byte. */
int nvfp4_selftest_e2m1_encode(const float* y, uint8_t* hw_codes, uint8_t* sw_codes, int64_t n,
                               void* stream);

/* Every non-NaN binary32 pattern: adds to *mismatches (device, must start at 0) the count
 * where the conversion instruction and the software encoder differ, and stores up to 16
 * offending bit patterns in first16 (device, 16 entries). */
int nvfp4_selftest_e2m1_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                   void* stream);

/* Every pair (bf16 significand of x with x in [1, 4), binary32 significand of d in
 * [1, 2)): adds to *mismatches (device, starts at 0) the count where the quantizer's
 * reciprocal-plus-correction quotient differs from IEEE x / d; up to 8 (x, d) bit-pattern
 * pairs land in first16 (device, 16 entries). */
int nvfp4_selftest_division(unsigned long long* mismatches, uint32_t* first16, void* stream);

/* For each amax[i] (binary32, >= 0): codes[i] = the block scale code the quantizer
 * picks under global_scale, d[i] = RN(decode(code) * global_scale). */
int nvfp4_selftest_block_scale(const float* amax, float global_scale, uint8_t* codes, float* d,
                               int64_t n, void* stream);

/* Every binary32 pattern except NaN and Inf, clamped to [-448, 448] as the MXFP8
 * quantizer does: adds to *mismatches (device, starts at 0) the count where the gfx950 fp8
 * conversion and the software E4M3 encoder (sign copied, nearest, ties to even) differ;
 * up to 16 offending patterns land in first16 (device, 16 entries). */
int nvfp4_selftest_mxfp8_e4m3_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                         void* stream);

/* The same for the bf8 (E5M2) conversion of the MXFP8 quantizer: every non-NaN, non-Inf
 * binary32 pattern clamped to [-57344, 57344], converted by the hardware and by the
 * software E5M2 encoder (nearest, ties to even, saturating, sign copied). */
int nvfp4_selftest_mxfp8_e5m2_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                         void* stream);

/* The GEMM epilogues' packed fp32 -> bf16 conversion (gfx950 v_cvt_pk_bf16_f32) against
 * round-to-nearest-even on the bit pattern, for every binary32 pattern except NaN (each in
 * both halves of the instruction): adds the mismatch count to *mismatches (device,
 * starts at 0); up to 16 offending patterns land in first16 (device, 16 entries). */
int nvfp4_selftest_bf16_exhaustive(unsigned long long* mismatches, uint32_t* first16,
                                   void* stream);

/* The GEMM's operand decode: packed[nbytes] holds 2*nbytes E2M1 codes (low nibble
 * first); scales[nbytes / 4] holds one E4M3 code per 4 packed bytes. Writes 2*nbytes
 * f16 bit patterns of code value * scale to hw_f16 (conversion-instruction decode) and
 * sw_f16 (byte-table decode). nbytes must be a multiple of 4 and both outputs 16-byte
 * aligned, else NVFP4_ERROR_HIP (hipErrorInvalidValue). */
int nvfp4_selftest_decode(const uint8_t* packed, const uint8_t* scales, uint16_t* hw_f16,
                          uint16_t* sw_f16, int64_t nbytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_SELFTEST_H_ */
