"""Plain, slow CPU oracle for the MXFP8 path (NumPy, vectorised).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path (the HIP
library under ``nvfp4_block_scaled_02_amd/`` and its Python binding) never imports, calls
or links anything here, and nothing here imports the product path.

What the path computes, as the pages state it
---------------------------------------------
* zubnet.ai, "NVIDIA FP4 format: diffusion model 1.68x speedup" (Hindi), paragraph 1:
  MXFP8 is the second microscaling format the page measures (1.26x end to end on
  Blackwell); it follows the Open Compute Project standard, with 8-bit E4M3/E5M2
  elements in 32-element blocks that share one higher-precision scale.

Readings taken where the pages are silent (the page names the OCP microscaling
standard; these follow its format definition, and are conventions of this library)
---------------------------------------------------------------------------------------
* Element type E4M3 (OCP "FN": no Inf, max 448). Block = 32 consecutive elements along
  K of a row-major [rows, K] tensor (K % 32 == 0); codes stored one byte per element,
  row-major [rows, K]; scales stored row-major [rows, K/32].
* The shared scale is an E8M0 byte: value 2^(byte - 127); byte 0xFF (NaN) is never
  produced.
* Shared exponent of a block: e = floor(log2(amax)) - 8, where 8 is the exponent of
  E4M3's largest normal (448 = 1.75 * 2^8), clamped to [-127, 127]. An all-zero block
  takes e = -127 (byte 0).
* Elements: y = x / 2^e (exact), code = the E4M3 value nearest to |y| (ties to the even
  code; values above 448 saturate to 448, never NaN), with the sign of x copied, so -0
  encodes as 0x80.
* GEMM: out[m, n] = bf16(sum_k a[m,k] w[n,k]) with a = e4m3(code) * 2^(e of its block)
  and w likewise; no tensor-level scale. Any summation order is acceptable; the result
  must satisfy |out - ref| <= 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp(ref), the NVFP4
  GEMM's bound.

Parity unpinned (conventions with no external reference): the byte layouts, the scale
byte of an all-zero block and the treatment of elements above 448 after scaling
(saturation). They are fixed here and by the tests, not by the pages.
"""
from __future__ import annotations

import numpy as np

from .nvfp4_oracle import _E4M3_POS, _nearest_code_ties_even, bf16_bits_to_f32, e4m3_decode

BLOCK = 32
E4M3_EMAX = 8  # exponent of the largest normal E4M3 value, 448 = 1.75 * 2^8
E8M0_BIAS = 127


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - E8M0_BIAS))


def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exact (from the binary exponent, no log)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1  # frexp: a = m * 2^e with m in [0.5, 1)


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """Block exponent e (scale 2^e) for block maxima ``amax`` >= 0."""
    a = np.asarray(amax, dtype=np.float64)
    e = floor_log2(np.where(a > 0, a, 1.0)) - E4M3_EMAX
    e = np.clip(e, -E8M0_BIAS, E8M0_BIAS)
    return np.where(a > 0, e, -E8M0_BIAS).astype(np.int64)


def e4m3_encode_signed(y: np.ndarray) -> np.ndarray:
    """E4M3 byte nearest to each finite y (ties to even, saturating at +-448, sign of y
    copied, -0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)):
        raise ValueError("e4m3_encode_signed expects finite inputs")
    mag = _nearest_code_ties_even(np.abs(y), _E4M3_POS).astype(np.uint8)
    return np.where(np.signbit(y), mag | np.uint8(0x80), mag).astype(np.uint8)


def quantize(x_bits: np.ndarray, *, chunk_rows: int = 1024):
    """MXFP8 (E4M3, 32-element blocks, E8M0 scales) of a bf16 tensor [rows, K].

    Returns ``(codes uint8 [rows, K], scales uint8 [rows, K/32])``.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((R, K), dtype=np.uint8)
    scales = np.empty((R, K // BLOCK), dtype=np.uint8)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        x = bf16_bits_to_f32(x_bits[r0:r1]).astype(np.float64).reshape(r1 - r0, K // BLOCK, BLOCK)
        amax = np.abs(x).max(axis=-1)
        e = shared_exponent(amax)
        y = np.ldexp(x, -e[..., None])  # exact: scaling by a power of two
        codes[r0:r1] = e4m3_encode_signed(y).reshape(r1 - r0, K)
        scales[r0:r1] = (e + E8M0_BIAS).astype(np.uint8)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values e4m3(code) * 2^(e of the block); [rows, K]."""
    R, K = codes.shape
    v = e4m3_decode(codes).reshape(R, K // BLOCK, BLOCK)
    return (v * e8m0_decode(scales)[..., None]).reshape(R, K)


def gemm_ref(a_codes, a_scales, w_codes, w_scales, *, with_abs: bool = True):
    """Reference MXFP8 product out = A_hat @ W_hat^T in float64.

    A is [M, K] activations, W is [N, K] weights, both MXFP8. Each decoded product is
    exact in float64 (4-bit significands); the float64 sum differs from the exact sum by
    far less than the acceptance bound. Returns ``(ref, absref)``.
    """
    A = dequantize(a_codes, a_scales)
    W = dequantize(w_codes, w_scales)
    ref = A @ W.T
    absref = np.abs(A) @ np.abs(W).T if with_abs else None
    return ref, absref

