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
* Element types: E4M3 (OCP "FN": 4 exponent bits, bias 7, 3 mantissa bits, no Inf,
  max 448 = 1.75 * 2^8) and E5M2 (5 exponent bits, bias 15, 2 mantissa bits, IEEE-like
  Inf/NaN at exponent field 31, max finite 57344 = 1.75 * 2^15). Block = 32 consecutive
  elements along K of a row-major [rows, K] tensor (K % 32 == 0); codes stored one
  byte per element, row-major [rows, K]; scales stored row-major [rows, K/32].
* The shared scale is an E8M0 byte: value 2^(byte - 127); byte 0xFF (NaN) is never
  produced.
* Shared exponent of a block: e = floor(log2(amax)) - emax, where emax is the exponent
  of the element type's largest normal (8 for E4M3, 15 for E5M2), clamped to
  [-127, 127]. An all-zero block takes e = -127 (byte 0).
* Elements: y = x / 2^e (exact), code = the finite value of the element type nearest to
  |y| (ties to the even code; values above the largest finite value saturate to it,
  never Inf or NaN), with the sign of x copied, so -0 encodes as 0x80.
* GEMM: out[m, n] = bf16(sum_k a[m,k] w[n,k]) with a = elem(code) * 2^(e of its block)
  and w likewise (each operand with its own element type); no tensor-level scale. Any
  summation order is acceptable; the result must satisfy
  |out - ref| <= 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp(ref), the NVFP4 GEMM's bound.

Parity unpinned (conventions with no external reference): the byte layouts, the scale
byte of an all-zero block and the treatment of elements above the largest finite value
after scaling (saturation). They are fixed here and by the tests, not by the pages.
"""
from __future__ import annotations

import numpy as np

from .nvfp4_oracle import _E4M3_POS, _nearest_code_ties_even, bf16_bits_to_f32, e4m3_decode

BLOCK = 32
E4M3_EMAX = 8  # exponent of the largest normal E4M3 value, 448 = 1.75 * 2^8
E5M2_EMAX = 15  # exponent of the largest normal E5M2 value, 57344 = 1.75 * 2^15
E8M0_BIAS = 127


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """Value of E5M2 bytes: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits.

    Exponent field 0 is subnormal (m * 2^-16); field 31 is Inf (m == 0) or NaN.
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    e = (c >> 2) & 0x1F
    m = c & 3
    mag = np.where(e == 0, m * 2.0**-16, np.exp2(e - 15.0) * (1.0 + m / 4.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where((c >> 7) & 1, -mag, mag)


# The finite non-negative E5M2 values in code order (codes 0x00..0x7B); increasing.
_E5M2_POS = e5m2_decode(np.arange(0x7C))

# element type -> (decode, increasing finite non-negative table, emax)
ELEMENTS = {
    "e4m3": (e4m3_decode, _E4M3_POS, E4M3_EMAX),
    "e5m2": (e5m2_decode, _E5M2_POS, E5M2_EMAX),
}


def _elem(elem: str):
    if elem not in ELEMENTS:
        raise ValueError(f"unknown MXFP8 element type {elem!r}")
    return ELEMENTS[elem]


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - E8M0_BIAS))


def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exact (from the binary exponent, no log)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1  # frexp: a = m * 2^e with m in [0.5, 1)


def shared_exponent(amax: np.ndarray, elem: str = "e4m3") -> np.ndarray:
    """Block exponent e (scale 2^e) for block maxima ``amax`` >= 0."""
    emax = _elem(elem)[2]
    a = np.asarray(amax, dtype=np.float64)
    e = floor_log2(np.where(a > 0, a, 1.0)) - emax
    e = np.clip(e, -E8M0_BIAS, E8M0_BIAS)
    return np.where(a > 0, e, -E8M0_BIAS).astype(np.int64)


def encode_signed(y: np.ndarray, elem: str = "e4m3") -> np.ndarray:
    """Byte of the element type nearest to each finite y (ties to even, saturating at the
    largest finite value, sign of y copied, -0 -> 0x80)."""
    table = _elem(elem)[1]
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)):
        raise ValueError("encode_signed expects finite inputs")
    mag = _nearest_code_ties_even(np.abs(y), table).astype(np.uint8)
    return np.where(np.signbit(y), mag | np.uint8(0x80), mag).astype(np.uint8)


def e4m3_encode_signed(y: np.ndarray) -> np.ndarray:
    """E4M3 byte nearest to each finite y (ties to even, saturating at +-448, sign of y
    copied, -0 -> 0x80)."""
    return encode_signed(y, "e4m3")


def quantize(x_bits: np.ndarray, *, elem: str = "e4m3", chunk_rows: int = 1024):
    """MXFP8 (E4M3 or E5M2 elements, 32-element blocks, E8M0 scales) of a bf16 tensor
    [rows, K].

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
        e = shared_exponent(amax, elem)
        y = np.ldexp(x, -e[..., None])  # exact: scaling by a power of two
        codes[r0:r1] = encode_signed(y, elem).reshape(r1 - r0, K)
        scales[r0:r1] = (e + E8M0_BIAS).astype(np.uint8)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, elem: str = "e4m3") -> np.ndarray:
    """float64 values elem(code) * 2^(e of the block); [rows, K]."""
    R, K = codes.shape
    v = _elem(elem)[0](codes).reshape(R, K // BLOCK, BLOCK)
    return (v * e8m0_decode(scales)[..., None]).reshape(R, K)


def gemm_ref(a_codes, a_scales, w_codes, w_scales, *, a_elem: str = "e4m3",
             w_elem: str = "e4m3", with_abs: bool = True):
    """Reference MXFP8 product out = A_hat @ W_hat^T in float64.

    A is [M, K] activations, W is [N, K] weights, both MXFP8 (element types a_elem and
    w_elem). Each decoded product is exact in float64 (at most 4-bit significands); the
    float64 sum differs from the exact sum by far less than the acceptance bound.
    Returns ``(ref, absref)``.
    """
    A = dequantize(a_codes, a_scales, a_elem)
    W = dequantize(w_codes, w_scales, w_elem)
    ref = A @ W.T
    absref = np.abs(A) @ np.abs(W).T if with_abs else None
    return ref, absref

