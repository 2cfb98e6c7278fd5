/*
 * libnvfp4 -- NVFP4 W4A4 linear layers on AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every entry point takes plain pointers and sizes; no C++ types cross it and no
 * exception escapes it. Device buffers and streams belong to the caller; the library
 * allocates nothing, keeps no per-call state and never synchronises the host.
 *
 * The format (what a stored tensor is):
 *   - "BFL (fp8r / nvfp4)" (Hugging Face diffusers docs), scheme list, item nvfp4: a
 *     quantized linear layer stores a packed E2M1 `weight` (two values per byte), E4M3
 *     block scales `weight_scale`, a global fp32 `weight_scale_2` and a calibrated fp32
 *     activation scale `input_scale`.
 *   - zubnet.ai, "NVIDIA FP4 format: diffusion model 1.68x speedup", paragraph 1:
 *     microscaling, one shared scale per small block; NVFP4 = E2M1 with 16-element
 *     blocks.
 *   - "BFL (fp8r / nvfp4)", Kernels table, nvfp4 row: activations are quantized at run
 *     time and fed, with the stored weights, to one fused FP4 GEMM.
 *
 * Conventions of this library (the pages do not fix them):
 *   - A tensor is row-major [rows, K], K % 16 == 0. Blocks are 16 consecutive elements
 *     along K. packed is uint8 [rows, K/2]: byte j of a row holds element 2j in its low
 *     nibble and element 2j+1 in its high nibble. scales is uint8 [rows, K/16] of OCP
 *     E4M3 ("FN") codes, never negative or NaN, at most 0x7E (448).
 *   - An E2M1 code is sign<<3 | magnitude code; magnitudes 0..7 are
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}. Negative zero is code 0x8.
 *   - Global scales are host fp32 in the dequantise direction:
 *     value = e2m1(code) * e4m3(scale) * global.
 *   - bf16 tensors are raw 16-bit storage. Weights are [N, K] (a linear layer's
 *     layout); out = x * W^T is [M, N] bf16, row-major.
 *   - Quantization rounding (every step IEEE binary32, round to nearest even): per block,
 *     amax = max|x|; s = E4M3(RN(amax / RN(6 * global))) with ties to the even code and
 *     saturation at 448; d = RN(s * global); code_i = E2M1(RN(|x_i| / d)) with ties to
 *     the even code, saturation at 6 and the sign of x_i copied (d == 0 gives magnitude 0).
 *   - GEMM: out = bf16_RNE(RN(alpha * sum_k a_k w_k)) with the decoded (E2M1 x E4M3)
 *     operands and alpha = RN(a_global * w_global); the products are exact and
 *     accumulate in fp32. Where that alpha would not be a normal fp32 (valid global
 *     scales multiply to anything in [2^-180, 2^180]) the product is applied as m * 2^e
 *     instead (m the rounded product of the two scales' frexp mantissas, 2^e by an exact
 *     ldexp). Any result within 2^-10 * sum_k |a_k w_k| (global scales included) + 1 bf16
 *     ulp of the exact value is correct; the library's result is deterministic for a
 *     given shape.
 *
 * Preconditions that are not checked (checking them would read the data):
 *   inputs are finite; buffers do not overlap; pointers are device memory of the
 *   current device (any HIP device pointer, including managed memory).
 *
 * Streams: `stream` is a hipStream_t passed as void*; NULL means the null stream.
 * Every compute call is asynchronous and stream-ordered. Calls are thread-safe.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 5

/* Status codes. All argument validation happens before any HIP call. */
typedef enum nvfp4_status {
  NVFP4_SUCCESS = 0,                  /* also returned for an empty problem (M == 0 or N == 0) */
  NVFP4_ERROR_INVALID_VALUE = 1,      /* null pointer; global scale not finite, <= 0, or
                                         outside [2^-90, 2^90]. The range is a restriction
                                         of this library beyond "finite and > 0": inside it
                                         the quantizer's reciprocal-plus-correction
                                         divisions are exact (their residuals never
                                         underflow); any bf16 tensor with amax in
                                         [2^-78, 2^101] calibrates into it */
  NVFP4_ERROR_INVALID_SHAPE = 2,      /* negative size, K < 16, K % 16 != 0, size overflow */
  NVFP4_ERROR_MISALIGNED = 3,         /* x, packed, out or workspace not 16-byte aligned;
                                         scales not 4-byte aligned */
  NVFP4_ERROR_WORKSPACE = 4,          /* workspace smaller than nvfp4_linear_workspace_bytes */
  NVFP4_ERROR_UNSUPPORTED_DEVICE = 5, /* no HIP device, or the current device is not gfx950 */
  NVFP4_ERROR_HIP = 6,                /* a HIP call failed; see nvfp4_last_hip_error() */
  NVFP4_ERROR_TOO_LARGE = 7           /* nvfp4_linear_noalloc: the problem's workspace exceeds
                                         the library's static scratch (32 MiB) */
} nvfp4_status;

/*
 * Version of this ABI (NVFP4_ABI_VERSION). A binding must refuse a mismatch, as the pages'
 * FP4 kernel package refuses to import when its two parts differ in version ("BFL (fp8r /
 * nvfp4)", paragraph under the Kernels table: the Python and the prebuilt-kernel packages
 * have to be installed at the same version). The Python binding of this library checks it
 * on load and raises on a mismatch.
 */
int nvfp4_abi_version(void);

/* Static string naming a status code (never NULL). */
const char* nvfp4_status_string(int status);

/* hipError_t of the last NVFP4_ERROR_HIP returned on the calling thread (0 if none). */
int nvfp4_last_hip_error(void);

/*
 * Runtime activation (or offline weight) quantization, the counterpart of the pages'
 * nvfp4_quantize ("BFL (fp8r / nvfp4)", Kernels table, nvfp4 row).
 *   x_bf16       device, bf16 [M, K], 16-byte aligned, read only
 *   M, K         rows and columns; M >= 0, K >= 16, K % 16 == 0
 *   global_scale fp32 per-tensor scale (input_scale for activations, weight_scale_2 for
 *                weights), finite, in [2^-90, 2^90] (any bf16 tensor with amax in
 *                [2^-78, 2^101] calibrates into this range)
 *   packed       device, uint8 [M, K/2], 16-byte aligned, written
 *   scales       device, uint8 [M, K/16], 4-byte aligned, written
 * The output is bit-exact to the rounding rule in the header comment.
 */
int nvfp4_quantize(const void* x_bf16, int64_t M, int64_t K, float global_scale,
                   void* packed, void* scales, void* stream);

/*
 * Block-scaled W4A4 GEMM, the counterpart of the pages' mm_fp4 ("BFL (fp8r / nvfp4)",
 * Kernels table, nvfp4 row): out[M, N] = a_global * w_global * A_hat[M, K] W_hat[N, K]^T.
 *   a_packed, a_scales  device, activations in NVFP4 layout [M, K/2], [M, K/16]
 *   w_packed, w_scales  device, weights in NVFP4 layout [N, K/2], [N, K/16]
 *   a_global_scale, w_global_scale  fp32, finite, in [2^-90, 2^90]
 *   out_bf16            device, bf16 [M, N], 16-byte aligned, written
 * Packed operands must be 16-byte aligned, scales 4-byte aligned.
 */
int nvfp4_gemm(const void* a_packed, const void* a_scales, float a_global_scale,
               const void* w_packed, const void* w_scales, float w_global_scale,
               int64_t M, int64_t N, int64_t K, void* out_bf16, void* stream);

/* Kernels nvfp4_gemm chooses among (reported by nvfp4_gemm_plan). */
typedef enum {
  NVFP4_GEMM_TILE256 = 0, /* 256 x 256 output tiles, direct-to-LDS loads (K % 128 == 0) */
  NVFP4_GEMM_FIT = 1,     /* 288 x 192 output tiles (K % 128 == 0): 4608-row activations
                             and FLUX widths split into whole multiples of 256 tiles */
  NVFP4_GEMM_SPLITK = 2,  /* K split over a workgroup's waves: short activations */
  NVFP4_GEMM_GENERIC = 3, /* 256 x 256 tiles, register-staged loads: any K % 16 == 0 */
  NVFP4_GEMM_TILE128 = 4, /* 128 x 192 output tiles (K % 128 == 0): activations of a few
                             hundred to a few thousand rows */
  NVFP4_GEMM_TILE128X128 = 5, /* 128 x 128 output tiles (K % 128 == 0): more tiles, where
                                 the larger ones would leave compute units idle */
  NVFP4_GEMM_TILE128X64 = 6,   /* 128 x 64 output tiles (K % 128 == 0): more still, for a few
                                 hundred rows */
  NVFP4_GEMM_WSPLIT64 = 7,     /* 64 x 64 output tiles whose four waves split K (K % 512 == 0):
                                 a few hundred activation rows against a narrow weight */
  NVFP4_GEMM_WSPLIT128 = 8,    /* 128 x 128 output tiles, two row bands of two waves that
                                 split K (K % 256 == 0): about a thousand rows, long K */
  NVFP4_GEMM_GEMV16 = 9        /* at most 16 activation rows, or 32 where N <= 16 x the
                                 compute units (K % 256 == 0): 4 to 16 weight rows per
                                 workgroup, 16 x 16 x 32 MFMAs, the weights' read spread
                                 over every compute unit */
} nvfp4_gemm_kernel;

/*
 * The kernel nvfp4_gemm launches for an M x N x K product on a device with num_cus
 * compute units (<= 0: 256, an MI355X), given 16-byte aligned packed operands and 4-byte
 * aligned scales. Host only: no device call. Writes an nvfp4_gemm_kernel value to
 * *kernel; returns NVFP4_ERROR_INVALID_VALUE for a null kernel pointer and
 * NVFP4_ERROR_INVALID_SHAPE for shapes nvfp4_gemm rejects.
 */
int nvfp4_gemm_plan(int64_t M, int64_t N, int64_t K, int num_cus, int* kernel);

/*
 * W4A16 GEMM: NVFP4 weights, bf16 activations left unquantized, the pages' path for
 * hardware without the fused FP4 kernel ("BFL (fp8r / nvfp4)", text under the Kernels
 * table: the weights are dequantized to the compute dtype and the layer runs as an
 * ordinary linear, so results differ slightly from the W4A4 path).
 *   out = bf16_RNE(w_global * sum_k x_k w_k) with w_k = E2M1 x E4M3 decoded exactly; the
 *   products are exact and accumulate in fp32; any result within
 *   2^-10 * sum_k |x_k w_k| (global scale included) + 1 bf16 ulp of the exact value is
 *   correct, and the library's result is deterministic for a given shape.
 *   x_bf16              device, bf16 [M, K], 16-byte aligned, read only
 *   w_packed, w_scales  device, weights in NVFP4 layout [N, K/2] (16-byte aligned),
 *                       [N, K/16] (4-byte aligned)
 *   w_global_scale      fp32, finite, in [2^-90, 2^90]
 *   K                   K % 32 == 0 and K <= 2^22 (else NVFP4_ERROR_INVALID_SHAPE)
 *   out_bf16            device, bf16 [M, N], 16-byte aligned, written
 */
int nvfp4_gemm_w4a16(const void* x_bf16, const void* w_packed, const void* w_scales,
                     float w_global_scale, int64_t M, int64_t N, int64_t K, void* out_bf16,
                     void* stream);

/* Kernels nvfp4_gemm_w4a16 chooses among (reported by nvfp4_gemm_w4a16_plan). */
typedef enum {
  NVFP4_W4A16_SPLITK = 0,  /* K split over a workgroup's waves: at most 64 rows, or K % 64 != 0 */
  NVFP4_W4A16_FIT = 1,     /* 288 x 192 output tiles (K % 64 == 0) */
  NVFP4_W4A16_TILE256 = 2, /* 256 x 256 output tiles (K % 64 == 0) */
  NVFP4_W4A16_WIDE = 3,    /* 224 x 256 output tiles with the waves side by side along N
                              (K % 64 == 0): each weight group decoded once per tile */
  NVFP4_W4A16_WIDE128X256 = 4, /* the same layout on 128 x 256, */
  NVFP4_W4A16_WIDE96X256 = 5,  /* 96 x 256, */
  NVFP4_W4A16_WIDE128X128 = 6, /* 128 x 128 */
  NVFP4_W4A16_WIDE64X128 = 7, /* and 64 x 128 tiles: medium and short activations */
  NVFP4_W4A16_GEMV16 = 8       /* at most 16 activation rows, or 32 where N <= 16 x the
                                  compute units (K % 256 == 0): 4 to 16 weight rows per
                                  workgroup on 16 x 16 x 32 bf16 MFMAs */
} nvfp4_w4a16_kernel;

/*
 * The kernel nvfp4_gemm_w4a16 launches for an M x N x K product on a device with num_cus
 * compute units (<= 0: 256, an MI355X). Host only: no device call. Writes an
 * nvfp4_w4a16_kernel value to *kernel; returns NVFP4_ERROR_INVALID_VALUE for a null
 * kernel pointer and NVFP4_ERROR_INVALID_SHAPE for shapes nvfp4_gemm_w4a16 rejects.
 */
int nvfp4_gemm_w4a16_plan(int64_t M, int64_t N, int64_t K, int num_cus, int* kernel);

/*
 * MXFP8 (OCP microscaling) path: the second microscaling format of the zubnet.ai page
 * (paragraph 1: Open Compute Project standard, 8-bit E4M3/E5M2 elements, 32-element
 * blocks sharing one scale). Conventions of this library (the page names the OCP
 * standard; these follow its format definition):
 *   - elements are one byte each, row-major [rows, K], of either OCP type:
 *     E4M3 ("FN": bias 7, no Inf, largest 448 = 1.75 * 2^8) or E5M2 (bias 15, Inf/NaN at
 *     exponent field 31, largest finite 57344 = 1.75 * 2^15);
 *   - each 32-element block along K shares an E8M0 scale byte (value 2^(byte - 127),
 *     0xFF never produced), row-major [rows, K/32];
 *   - quantization: e = floor(log2(amax)) - emax clamped to [-127, 127], emax = 8 for
 *     E4M3 and 15 for E5M2 (all-zero block: e = -127, byte 0); element = the value of the
 *     element type nearest to x / 2^e, ties to even, saturating at its largest finite
 *     value (never Inf or NaN), sign copied (-0 -> 0x80);
 *   - GEMM: out = bf16_RNE(sum_k a_k w_k) with a_k, w_k the decoded values, no tensor
 *     scale; any result within 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp of the exact value is
 *     correct and the library's result is deterministic for a given shape.
 *
 * nvfp4_mxfp8_quantize: x_bf16 [M, K] (16-byte aligned) -> codes uint8 [M, K] (16-byte
 * aligned) and scales uint8 [M, K/32]. K % 32 == 0. Bit-exact to the rule above.
 */
int nvfp4_mxfp8_quantize(const void* x_bf16, int64_t M, int64_t K, void* codes, void* scales,
                         void* stream);

/*
 * nvfp4_mxfp8_gemm: out_bf16 [M, N] = A_hat [M, K] W_hat [N, K]^T with both operands MXFP8
 * (activations a_codes/a_scales, weights w_codes/w_scales as produced by
 * nvfp4_mxfp8_quantize). K % 128 == 0 and (max(M, N) + 256) * K < 2^31, else
 * NVFP4_ERROR_INVALID_SHAPE; codes and out 16-byte aligned, scales 4-byte aligned.
 * Runs on gfx950's block-scaled fp8 MFMA, which applies the E8M0 scales itself.
 */
int nvfp4_mxfp8_gemm(const void* a_codes, const void* a_scales, const void* w_codes,
                     const void* w_scales, int64_t M, int64_t N, int64_t K, void* out_bf16,
                     void* stream);

/* MXFP8 element types (the `element` arguments below). */
typedef enum { NVFP4_MX_E4M3 = 0, NVFP4_MX_E5M2 = 1 } nvfp4_mx_element;

/*
 * nvfp4_mxfp8_quantize with the element type chosen (NVFP4_MX_E4M3 is
 * nvfp4_mxfp8_quantize); any other value returns NVFP4_ERROR_INVALID_VALUE.
 */
int nvfp4_mxfp8_quantize_elem(const void* x_bf16, int64_t M, int64_t K, int element,
                              void* codes, void* scales, void* stream);

/*
 * nvfp4_mxfp8_gemm with each operand's element type chosen (E4M3 x E4M3 is
 * nvfp4_mxfp8_gemm): the block-scaled MFMA takes the two operand formats separately, so
 * E4M3 and E5M2 operands mix freely. Other requirements as nvfp4_mxfp8_gemm; an unknown
 * element type returns NVFP4_ERROR_INVALID_VALUE.
 */
int nvfp4_mxfp8_gemm_elem(const void* a_codes, const void* a_scales, int a_element,
                          const void* w_codes, const void* w_scales, int w_element, int64_t M,
                          int64_t N, int64_t K, void* out_bf16, void* stream);

/*
 * Rowwise FP8 ("fp8r") path: the other scheme of the "BFL (fp8r / nvfp4)" page (scheme
 * list, fp8r item: an E4M3 weight and one fp32 weight_scale per row, activations quantized
 * to E4M3 per row at run time; Kernels table, fp8r row: a scaled matmul with rowwise
 * scales). Conventions of this library where the page is silent:
 *   - scale of a row: s = RN32(amax / 448) (448 = the largest E4M3 value), 1.0 for an
 *     all-zero row; dequantize direction, x ~ e4m3(code) * s;
 *   - element: the E4M3 value nearest to RN32(x / s) (IEEE division), ties to even,
 *     clamped to +-448, sign copied (-0 -> 0x80);
 *   - layouts: codes uint8 [rows, K] row-major, scales fp32 [rows];
 *   - GEMM: out = bf16_RNE(s_a[m] * s_w[n] * sum_k e4m3(a[m,k]) e4m3(w[n,k])); any result
 *     within 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp of the exact value is correct and the
 *     library's result is deterministic for a given shape. The epilogue evaluates
 *     RN(RN(sum * s_a[m]) * s_w[n]) in fp32, so the bound assumes the intermediate
 *     sum * s_a[m] stays inside fp32's normal range: an activation row with amax above
 *     about 2^99 can overflow it, and a row of bf16 subnormals paired with a weight row
 *     above about 2^20 can lose precision in it.
 *
 * nvfp4_fp8r_quantize: x_bf16 [M, K] (16-byte aligned) -> codes uint8 [M, K] (16-byte
 * aligned) and scales fp32 [M] (4-byte aligned). K >= 16, K % 16 == 0. Bit-exact to the
 * rule above (weights are quantized offline with the same call).
 */
int nvfp4_fp8r_quantize(const void* x_bf16, int64_t M, int64_t K, void* codes, void* scales,
                        void* stream);

/*
 * nvfp4_fp8r_gemm: out_bf16 [M, N] = diag(a_scales) Qa Qw^T diag(w_scales) with activations
 * a_codes [M, K] / a_scales fp32 [M] and weights w_codes [N, K] / w_scales fp32 [N] as
 * produced by nvfp4_fp8r_quantize. K % 128 == 0 and (max(M, N) + 256) * K < 2^31, else
 * NVFP4_ERROR_INVALID_SHAPE; codes and out 16-byte aligned, scales 4-byte aligned. Runs
 * on gfx950's block-scaled fp8 MFMA with unit block scales; the row and column scales are
 * applied in the epilogue.
 */
int nvfp4_fp8r_gemm(const void* a_codes, const void* a_scales, const void* w_codes,
                    const void* w_scales, int64_t M, int64_t N, int64_t K, void* out_bf16,
                    void* stream);

/*
 * Whether nvfp4_linear (and nvfp4_linear_devgs) run an M x N x K product as one kernel:
 * the short-activation GEMM that nvfp4_gemm would run (the 16-row kernel, or split-K)
 * first quantizing the bf16 activations into its LDS (for at most 32 rows and 24576
 * elements on the 16-row kernel, 16384 on split-K, where repeating that quantization in
 * every workgroup along N costs less than a second launch), instead of the quantize
 * kernel followed by nvfp4_gemm. num_cus as in nvfp4_gemm_plan. Host only.
 * Writes 1 (one kernel) or 0 (two) to *fused; NVFP4_ERROR_INVALID_VALUE for a null
 * pointer, NVFP4_ERROR_INVALID_SHAPE for shapes the linear rejects.
 */
int nvfp4_linear_plan(int64_t M, int64_t N, int64_t K, int num_cus, int* fused);

/* Workspace bytes nvfp4_linear needs for an [M, K] activation (packed + scales, each
 * rounded up to 256 bytes). Returns 0 for invalid shapes. */
size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * Fused linear: quantize x under a_global_scale into the workspace, then nvfp4_gemm,
 * both on `stream` ("BFL (fp8r / nvfp4)", Kernels table, nvfp4 row, fused-kernel column:
 * run-time activation quantization paired with the FP4 GEMM).
 *   x_bf16     device bf16 [M, K]
 *   workspace  device, >= nvfp4_linear_workspace_bytes(M, K) bytes, 256-byte aligned is
 *              best (16 required); it holds the quantized activations on return:
 *              packed [M, K/2] at offset 0, scales [M, K/16] at offset
 *              round_up(M*K/2, 256).
 * Other arguments as in nvfp4_quantize / nvfp4_gemm. Short activations (where
 * nvfp4_linear_plan reports 1) run as one kernel that quantizes inside the GEMM; the
 * workspace and the output are bit-identical to the two-kernel form either way.
 */
int nvfp4_linear(const void* x_bf16, float a_global_scale, const void* w_packed,
                 const void* w_scales, float w_global_scale, int64_t M, int64_t N, int64_t K,
                 void* out_bf16, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_linear without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). It runs the same kernels as nvfp4_linear, with their workspace in a static
 * device array of 32 MiB that the library holds on each device it is loaded on, for the
 * life of the process; it calls no allocator. Arguments as in nvfp4_linear, without
 * workspace and workspace_bytes; out is bit-identical to nvfp4_linear's for the same
 * inputs.
 *   - Limit: nvfp4_linear_workspace_bytes(M, K) <= 32 MiB (M * K up to about 59.6 million,
 *     e.g. [4608, 12288] or [18432, 3072] activations); larger problems return
 *     NVFP4_ERROR_TOO_LARGE before any HIP call.
 *   - Every call on a device shares that device's array, which keeps the last call's
 *     quantized activations. Calls that overlap in time on one device (on different
 *     streams, or from different threads without ordering) race on it and may produce
 *     wrong results; calls ordered on one stream are safe.
 *   - The first call on a device looks up the array's device address (once per device).
 */
int nvfp4_linear_noalloc(const void* x_bf16, float a_global_scale, const void* w_packed,
                         const void* w_scales, float w_global_scale, int64_t M, int64_t N,
                         int64_t K, void* out_bf16, void* stream);

/*
 * Calibration of a global scale (the pages' calibrated fp32 input_scale and the stored
 * weight_scale_2, "BFL (fp8r / nvfp4)", nvfp4 item).
 *
 * nvfp4_amax: amax_out[0] = max |x| over n bf16 values (0 for n == 0), computed on the
 * device and written to device memory (fp32). x_bf16 must be 16-byte aligned; amax_out
 * 4-byte aligned. Asynchronous.
 */
int nvfp4_amax(const void* x_bf16, int64_t n, float* amax_out, void* stream);

/* Host function: RN32(amax / (6 * 448)), or 1.0 when amax == 0. Returns a NaN for a
 * negative or non-finite amax. */
float nvfp4_global_scale_from_amax(float amax);

/*
 * Device-resident global scales: a dynamic activation scale ("calibrated" input_scale,
 * "BFL (fp8r / nvfp4)", nvfp4 item) computed and consumed on the device, with no host
 * round trip. All calls are asynchronous on `stream`; gs pointers are device memory,
 * 4-byte aligned.
 *
 * nvfp4_calibrate_device: gs_device[0] = RN32(amax / 2688) for the n bf16 values of
 * x_bf16 (16-byte aligned), clamped into [2^-90, 2^90]; 1.0 when amax == 0. Inside the
 * clamp range (any tensor with amax in [2^-78, 2^101]) this equals
 * nvfp4_global_scale_from_amax(amax). The clamp keeps extreme tensors quantizable.
 *
 * nvfp4_quantize_devgs: nvfp4_quantize with the global scale read from gs_device[0]
 * when the kernel runs (a value outside [2^-90, 2^90] is clamped into it; NaN and values
 * <= 0 read as 1.0). Bit-exact to nvfp4_quantize with that value.
 *
 * nvfp4_gemm_devgs: nvfp4_gemm with the two global scales read from a_gs_device[0] and
 * w_gs_device[0] when the kernel runs, each clamped as nvfp4_quantize_devgs clamps its
 * scale (into [2^-90, 2^90]; NaN and values <= 0 read as 1.0); bit-exact to nvfp4_gemm
 * with the two values so read.
 *
 * nvfp4_linear_devgs: nvfp4_linear with both global scales device-resident.
 */
int nvfp4_calibrate_device(const void* x_bf16, int64_t n, float* gs_device, void* stream);
int nvfp4_quantize_devgs(const void* x_bf16, int64_t M, int64_t K, const float* gs_device,
                         void* packed, void* scales, void* stream);
int nvfp4_gemm_devgs(const void* a_packed, const void* a_scales, const float* a_gs_device,
                     const void* w_packed, const void* w_scales, const float* w_gs_device,
                     int64_t M, int64_t N, int64_t K, void* out_bf16, void* stream);
int nvfp4_linear_devgs(const void* x_bf16, const float* a_gs_device, const void* w_packed,
                       const void* w_scales, const float* w_gs_device, int64_t M, int64_t N,
                       int64_t K, void* out_bf16, void* workspace, size_t workspace_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
