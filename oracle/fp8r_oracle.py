"""Plain, slow CPU oracle for the rowwise FP8 ("fp8r") path (NumPy, vectorised).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path (the HIP
library under ``nvfp4_block_scaled_02_amd/`` and its Python binding) never imports, calls
or links anything here, and nothing here imports the product path.

What the path computes, as the pages state it
---------------------------------------------
* "BFL (fp8r / nvfp4)", scheme list, ``fp8r`` item: every quantized linear layer stores an
  E4M3 ``weight`` and one fp32 ``weight_scale`` per row; activations are quantized to E4M3
  per row at run time.
* Same page, Kernels table, ``fp8r`` row: the product is a scaled matrix multiply with
  rowwise scales (one scale per activation row, one per weight row).

Readings taken where the pages are silent (conventions of this library)
-----------------------------------------------------------------------
* Scale of a row (weights and activations alike): s = RN32(amax / 448), amax the largest
  |x| of the row and 448 the largest E4M3 value, so the row's largest element maps to 448;
  an all-zero row takes s = 1. Dequantize direction: x ~ e4m3(code) * s.
* Elements: y = RN32(x / s) (IEEE binary32 division), clamped to [-448, 448] (only a
  rounding overshoot of the row maximum can exceed it), then the nearest E4M3 value with
  ties to the even code; the sign of x is copied, so -0 encodes as 0x80.
* Layouts: codes u8 [rows, K] row-major (one E4M3 byte per element), scales fp32 [rows].
* GEMM: out[m, n] = bf16(s_a[m] * s_w[n] * sum_k e4m3(a[m,k]) e4m3(w[n,k])): the scales
  leave the K-sum. Any summation order is acceptable; the result must satisfy the NVFP4
  GEMM's bound |out - ref| <= 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp(ref).

Parity unpinned (conventions with no external reference): the scale rule amax / 448 and
its all-zero case, the division (rather than a multiplication by a reciprocal) and the
layouts. They are fixed here and by the tests, not by the pages.
"""
from __future__ import annotations

import numpy as np

from .nvfp4_oracle import _E4M3_POS, _nearest_code_ties_even, bf16_bits_to_f32, e4m3_decode

E4M3_MAX = np.float32(448.0)


def row_scale(amax: np.ndarray) -> np.ndarray:
    """fp32 scale of each row from its fp32 amax: RN32(amax / 448), 1 for amax == 0."""
    a = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = a / E4M3_MAX  # IEEE binary32 division, correctly rounded
    return np.where(a > 0, s, np.float32(1.0)).astype(np.float32)


def e4m3_encode_signed(y: np.ndarray) -> np.ndarray:
    """E4M3 byte nearest to each finite |y| <= 448 (ties to even), sign of y copied."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > 448.0):
        raise ValueError("e4m3_encode_signed expects finite |y| <= 448")
    mag = _nearest_code_ties_even(np.abs(y), _E4M3_POS).astype(np.uint8)
    return np.where(np.signbit(y), mag | np.uint8(0x80), mag).astype(np.uint8)


def quantize(x_bits: np.ndarray, *, chunk_rows: int = 1024):
    """Rowwise FP8 of a bf16 tensor [rows, K] (bit patterns as uint16).

    Returns ``(codes uint8 [rows, K], scales float32 [rows])``.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    codes = np.empty((R, K), dtype=np.uint8)
    scales = np.empty((R,), dtype=np.float32)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        x = bf16_bits_to_f32(x_bits[r0:r1])  # float32, exact
        if np.any(~np.isfinite(x)):
            raise ValueError("inputs must be finite")
        amax = np.abs(x).max(axis=1) if K else np.zeros(r1 - r0, np.float32)
        s = row_scale(amax)
        y = x / s[:, None]  # float32 / float32: IEEE, correctly rounded
        y = np.clip(y, -E4M3_MAX, E4M3_MAX)
        codes[r0:r1] = e4m3_encode_signed(y)
        scales[r0:r1] = s
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values e4m3(code) * s (exact: a 4-bit significand times a binary32)."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def gemm_ref(a_codes, a_scales, w_codes, w_scales, *, with_abs: bool = True):
    """Reference product out = diag(s_a) (Qa Qw^T) diag(s_w) in float64.

    Qa Qw^T is exact in float64 for K < 2^17: every E4M3 value is a multiple of 2^-9 below
    2^9, so each product is a multiple of 2^-18 below 2^18, and every partial sum of at
    most K of them is a multiple of 2^-18 below K * 2^18 < 2^35, i.e. fewer than 2^53 units.
    The two scale factors then add two float64 roundings (2^-52 relative), far inside the
    acceptance bound. Returns ``(ref, absref)``.
    """
    if np.asarray(a_codes).shape[1] >= 1 << 17:
        raise ValueError("K >= 2^17: the float64 K-sum is no longer exact")
    qa = e4m3_decode(a_codes)
    qw = e4m3_decode(w_codes)
    sa = np.asarray(a_scales, dtype=np.float64)
    sw = np.asarray(w_scales, dtype=np.float64)
    acc = qa @ qw.T
    ref = acc * sa[:, None] * sw[None, :]
    absref = None
    if with_abs:
        absref = (np.abs(qa) @ np.abs(qw).T) * np.abs(sa)[:, None] * np.abs(sw)[None, :]
    return ref, absref

