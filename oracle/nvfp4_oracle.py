"""Plain, slow CPU oracle for the NVFP4 W4A4 linear path (NumPy, vectorised).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path (the
HIP library under ``nvfp4_block_scaled_02_amd/`` and its Python binding) never imports,
calls or links anything here, and nothing here imports the product path.

What the path computes, as the pages state it
---------------------------------------------
* "BFL (fp8r / nvfp4)" (Hugging Face diffusers docs, Korean build), scheme list, item
  ``nvfp4``: a quantized linear layer stores a packed E2M1 ``weight`` (two values per
  byte), E4M3 block scales ``weight_scale``, a global fp32 ``weight_scale_2`` and a
  calibrated fp32 activation scale ``input_scale``.
* Same page, Kernels table ("커널"), ``nvfp4`` row: activations are quantized at run time
  (``nvfp4_quantize``) and fed with the stored weights to a fused FP4 GEMM
  (``mm_fp4``); the output is a high-precision (here bf16) tensor.
* zubnet.ai, "NVIDIA FP4 format: diffusion model 1.68x speedup" (Hindi), paragraph 1:
  microscaling -- each small block of elements shares one higher-precision scale; NVFP4
  is E2M1 with 16-element blocks.

Readings taken where the pages are silent (each one is a convention of this library)
-------------------------------------------------------------------------------------
* Block = 16 consecutive elements along K, the last axis of a row-major [rows, K]
  tensor; scales are stored row-major [rows, K/16]; one byte holds elements 2j (low
  nibble) and 2j+1 (high nibble).
* Global scales are in the dequantise direction: x ~= e2m1 * e4m3_scale * global.
  Calibration: global = RN32(amax / (6 * 448)); an all-zero tensor gets 1.0.
* Quantize reading "R1": IEEE binary32, every operation correctly rounded to nearest
  even, in this order, per block of 16 values x_i:
    amax  = max_i |x_i|                       (exact)
    den   = RN32(6 * global)                  (once per tensor)
    s_raw = RN32(amax / den)
    S     = E4M3 code nearest to s_raw (ties to the even code; above 448 -> 448)
    d     = RN32(decode(S) * global)
    y_i   = RN32(|x_i| / d)                   (d == 0 -> magnitude code 0)
    code  = E2M1 magnitude nearest to y_i (ties to the even code; y >= 6 -> 6),
            with the sign bit of x_i copied (so -0.0 encodes as 0x8).
* GEMM: out[m, n] = bf16(a_gs * w_gs * sum_k a[m,k] w[n,k]) with a, w the decoded
  E2M1 * E4M3 values. Any summation order is acceptable; the result must satisfy
  |out - ref| <= 2^-10 * sum_k |a_k w_k| (global scales included) + 1 bf16 ulp(ref).

Parity unpinned (conventions with no external reference): the nibble order, the
scale layout, the code of negative zero and the exact fp32 operation order of R1.
They are fixed here and by the tests, not by the pages.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# Element and scale codecs
# --------------------------------------------------------------------------------------

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).

    Exponent field 0 is subnormal (m * 0.5); otherwise 2^(e-1) * (1 + m/2). The format
    has no Inf or NaN. E2M1 is NVFP4's element type (zubnet.ai page, paragraph 1;
    "BFL (fp8r / nvfp4)", ``nvfp4`` item).
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return np.where((c >> 3) & 1, -mag, mag)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3 ("FN") bytes: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; no Inf; max 448.
    E4M3 is the block-scale type ("BFL (fp8r / nvfp4)", ``nvfp4`` item).
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0**-9, np.exp2(e - 7.0) * (1.0 + m / 8.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where((c >> 7) & 1, -mag, mag)


# The finite non-negative E4M3 values in code order (codes 0x00..0x7E); increasing.
_E4M3_POS = e4m3_decode(np.arange(0x7F))
# The non-negative E2M1 magnitudes in code order (codes 0..7); increasing.
_E2M1_POS = e2m1_decode(np.arange(8))


def _nearest_code_ties_even(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the entry of the increasing ``table`` nearest to each v >= 0.

    Ties go to the even index (the code whose last mantissa bit is 0). Values above the
    last entry map to the last entry (saturation). Below the last entry, distances are
    taken in float64, where they are exact for float32 inputs and these
    short-significand tables.
    """
    v = np.asarray(v, dtype=np.float64)
    n = len(table)
    hi = np.clip(np.searchsorted(table, v, side="left"), 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    d_hi = np.abs(table[hi] - v)
    d_lo = np.abs(v - table[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    # Saturation: anything at or above the largest entry (including +inf) takes it.
    # Decided by comparison, not by distances, which stop being exact for huge v.
    idx = np.where(v >= table[-1], n - 1, idx)
    return idx.astype(np.uint8)


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    """E4M3 code of the finite E4M3 value nearest to each non-negative float32 ``s``.

    Ties go to the even code; anything above 448 saturates to 448 (0x7E), never NaN.
    """
    s = np.asarray(s, dtype=np.float32)
    if np.any(np.isnan(s)) or np.any(s < 0):
        raise ValueError("e4m3_encode expects non-negative, non-NaN inputs")
    return _nearest_code_ties_even(s, _E4M3_POS)


def e2m1_encode_magnitude(y: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code (0..7) nearest to each y >= 0; ties to even; y >= 6 -> 7."""
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.isnan(y)) or np.any(y < 0):
        raise ValueError("e2m1_encode_magnitude expects non-negative, non-NaN inputs")
    return _nearest_code_ties_even(y, _E2M1_POS)


# --------------------------------------------------------------------------------------
# bf16 storage helpers (raw uint16 bit patterns)
# --------------------------------------------------------------------------------------


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """bf16 unit in the last place at |v|: 2^(max(floor(log2|v|), -126) - 7); 2^-133 at 0."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # floor(log2) in float64 can be off by one next to powers of two; fix it exactly.
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 7.0), 2.0**-133)


# --------------------------------------------------------------------------------------
# Calibration (global scales)
# --------------------------------------------------------------------------------------


def global_scale_from_amax(amax: float) -> np.float32:
    """Per-tensor fp32 scale in the dequantise direction: RN32(amax / (6 * 448)).

    The pages name the stored fp32 ``weight_scale_2`` and the calibrated fp32
    ``input_scale`` ("BFL (fp8r / nvfp4)", ``nvfp4`` item) without the formula; this is
    the reading that maps the tensor's largest magnitude onto the largest E2M1 value
    (6) under the largest E4M3 scale (448). An all-zero tensor gets 1.0.
    """
    a = np.float32(amax)
    if not np.isfinite(a) or a < 0:
        raise ValueError("amax must be finite and non-negative")
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(2688.0))


def tensor_amax(x_bits: np.ndarray) -> np.float32:
    """Largest |x| of a bf16 tensor (exact in float32)."""
    xf = bf16_bits_to_f32(x_bits)
    if xf.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(xf)))


def global_scale(x_bits: np.ndarray) -> np.float32:
    """Calibrated global scale of a bf16 tensor: RN32(amax(|x|) / 2688)."""
    return global_scale_from_amax(tensor_amax(x_bits))


# --------------------------------------------------------------------------------------
# Quantize / dequantize
# --------------------------------------------------------------------------------------


def quantize(x_bits: np.ndarray, gs: float, *, chunk_rows: int = 1024):
    """NVFP4-quantize a bf16 tensor [R, K] (raw uint16 bits) under fp32 global ``gs``.

    Returns ``(packed uint8 [R, K/2], scales uint8 [R, K/16])`` following reading R1
    (see module docstring), step for step in float32 NumPy arithmetic, which is IEEE
    binary32 with correct rounding to nearest even for each operation.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("x must be 2-D [rows, K]")
    R, K = x_bits.shape
    if K % 16 != 0:
        raise ValueError("K must be a multiple of 16")
    gs32 = np.float32(gs)
    if not (np.isfinite(gs32) and gs32 > 0):
        raise ValueError("global scale must be finite and > 0")
    packed = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 16), dtype=np.uint8)
    den = np.float32(np.float32(6.0) * gs32)
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        xf = bf16_bits_to_f32(x_bits[r0:r1]).reshape(r1 - r0, K // 16, 16)
        if not np.all(np.isfinite(xf)):
            raise ValueError("inputs must be finite")
        ax = np.abs(xf)
        amax = ax.max(axis=-1)
        s_raw = (amax / den).astype(np.float32)
        S = e4m3_encode(s_raw)
        s = e4m3_decode(S).astype(np.float32)
        d = (s * gs32).astype(np.float32)
        dd = d[..., None]
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            y = (ax / np.where(dd == 0, np.float32(1.0), dd)).astype(np.float32)
        y = np.where(dd == 0, np.float32(0.0), y)
        mag = e2m1_encode_magnitude(y)
        code = (np.signbit(xf).astype(np.uint8) << 3) | mag
        packed[r0:r1] = (code[..., 0::2] | (code[..., 1::2] << 4)).reshape(r1 - r0, K // 2)
        scales[r0:r1] = S
    return packed, scales


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes (element 2j = low nibble of byte j)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def decode_blocks(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 [R, K]: e2m1(code) * e4m3(scale) per element, global scale NOT applied.

    Exact: the product has at most 2 + 4 significant bits.
    """
    q = e2m1_decode(unpack_codes(packed))
    s = e4m3_decode(scales)
    R, K = q.shape
    return (q.reshape(R, K // 16, 16) * s[..., None]).reshape(R, K)


def dequantize(packed: np.ndarray, scales: np.ndarray, gs: float) -> np.ndarray:
    """float64 [R, K] = e2m1 * e4m3 * global (exact in float64)."""
    return decode_blocks(packed, scales) * np.float64(np.float32(gs))


# --------------------------------------------------------------------------------------
# GEMM reference and acceptance test
# --------------------------------------------------------------------------------------


def gemm_ref(a_packed, a_scales, a_gs, w_packed, w_scales, w_gs, *, with_abs: bool = True,
             w_decoded=None):
    """Reference W4A4 product out = (A_hat @ W_hat^T) * a_gs * w_gs in float64.

    A is [M, K] activations, W is [N, K] weights (PyTorch Linear layout), both NVFP4.
    Each decoded product is exact in float64; the float64 sum differs from the exact
    sum by far less than the acceptance bound. Returns ``(ref, absref)`` where
    ``absref = (|A_hat| @ |W_hat|^T) * a_gs * w_gs`` feeds the tolerance (or ``None``).
    ``w_decoded``, if given, is ``decode_blocks(w_packed, w_scales)`` computed once by
    the caller for many calls over row chunks of A (a cache; nothing else changes).
    """
    A = decode_blocks(a_packed, a_scales)
    W = decode_blocks(w_packed, w_scales) if w_decoded is None else w_decoded
    g = np.float64(np.float32(a_gs)) * np.float64(np.float32(w_gs))
    ref = (A @ W.T) * g
    absref = (np.abs(A) @ np.abs(W).T) * g if with_abs else None
    return ref, absref


def gemm_exact_int(a_packed, a_scales, w_packed, w_scales) -> np.ndarray:
    """Exact integer form of sum_k a_k w_k (global scales excluded), as int64.

    a = (2q) * (s * 2^9) * 2^-10 with integer factors |2q| <= 12, s*2^9 <= 229376, so
    sum_k a_k w_k = S_int * 2^-20 exactly with |S_int| < 2^58 for K <= 12288.
    Returns S_int; callers multiply by 2^-20 (and the global scales).
    """
    def ints(packed, scales):
        q2 = np.rint(e2m1_decode(unpack_codes(packed)) * 2).astype(np.int64)
        s9 = np.rint(e4m3_decode(scales) * 512).astype(np.int64)
        R, K = q2.shape
        return (q2.reshape(R, K // 16, 16) * s9[..., None]).reshape(R, K)

    A = ints(a_packed, a_scales)
    W = ints(w_packed, w_scales)
    out = np.zeros((A.shape[0], W.shape[0]), dtype=np.int64)
    for k in range(A.shape[1]):  # exact int64 accumulation, no BLAS
        out += np.outer(A[:, k], W[:, k])
    return out


def gemm_tolerance(ref: np.ndarray, absref: np.ndarray) -> np.ndarray:
    """Per-element bound 2^-10 * sum_k |a_k w_k| + ulp_bf16(ref)."""
    return absref * 2.0**-10 + bf16_ulp(ref)


def check_gemm(out_bf16_bits: np.ndarray, ref: np.ndarray, absref: np.ndarray):
    """Compare a bf16 result (raw bits) with the reference; returns (ok, worst_ratio, n_bad)."""
    out = bf16_bits_to_f32(out_bf16_bits).astype(np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    tol = gemm_tolerance(ref, absref)
    err = np.abs(out - ref)
    bad = ~(err <= tol)  # NaN counts as bad
    ratio = np.where(tol > 0, err / tol, np.inf)
    ratio = np.where(np.isnan(ratio), np.inf, ratio)  # a NaN output is as bad as can be
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return (not bool(bad.any())), worst, int(bad.sum())


def w4a16_ref(x_bits, w_packed, w_scales, w_gs, *, with_abs: bool = True):
    """Dequantise-only product (bf16 activations kept unquantised), float64.

    The pages' fallback on devices without the fused kernel ("BFL (fp8r / nvfp4)",
    text under the Kernels table): weights are dequantised to the compute dtype every
    forward pass and the layer runs as an ordinary linear, so results differ slightly
    from the fused W4A4 kernel. Reading: the product uses the exactly decoded weights
    (q * s * w_gs); a bf16 x times a decoded weight is exact in float64, as is every
    partial sum far below the acceptance bound. Returns ``(ref, absref)`` with
    ``absref = |X| @ |W_hat|^T`` (global scale included) for the tolerance (or None).
    """
    X = bf16_bits_to_f32(x_bits).astype(np.float64)
    W = dequantize(w_packed, w_scales, w_gs)
    ref = X @ W.T
    absref = np.abs(X) @ np.abs(W).T if with_abs else None
    return ref, absref


def nvfp4_bytes(rows: int, K: int) -> int:
    """Storage of an NVFP4 tensor: packed codes + one scale byte per 16 + the fp32 global."""
    return rows * K // 2 + rows * K // 16 + 4
