"""Scalar, exact-arithmetic second oracle for NVFP4 quantisation (brute force).

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle/nvfp4_oracle.py``).

This module re-derives the quantiser from first principles with no NumPy arithmetic:
every value is a ``fractions.Fraction``; rounding to IEEE binary32 is written out
from its definition (nearest representable value, ties to the even significand,
gradual underflow, overflow to infinity); E4M3 scales and E2M1 magnitudes are chosen
by exhaustive search over every finite code. It pins the vectorised oracle on tiny
inputs: any slip there (a wrong tie rule, a dropped saturation, a wrong nibble) shows
up as a mismatch against this brute force.

Format facts used: E2M1 elements with one E4M3 scale per 16-element block and fp32
global scales ("BFL (fp8r / nvfp4)", ``nvfp4`` item; zubnet.ai page, paragraph 1).
The operation order is reading R1 (stated in ``oracle/nvfp4_oracle.py``).
"""
from __future__ import annotations

import struct
from fractions import Fraction

INF = float("inf")


def f32_bits_to_fraction(bits: int) -> Fraction:
    """Exact value of a finite binary32 bit pattern."""
    sign = -1 if (bits >> 31) & 1 else 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0xFF:
        raise ValueError("not finite")
    if e == 0:
        v = Fraction(m, 1 << 149)
    else:
        v = Fraction((1 << 23) | m) * Fraction(2) ** (e - 150)
    return sign * v


def float_to_fraction(x: float) -> Fraction:
    return Fraction(x)  # exact for any finite Python float


def rn32(q: Fraction):
    """Round a rational to the nearest binary32 value, ties to even significand.

    Returns a Fraction, or +/-INF on overflow. Subnormals have quantum 2^-149.
    """
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** 128:
        return sign * INF
    return sign * r


def fraction_to_f32_bits(v) -> int:
    """Bit pattern of a value that is exactly representable in binary32 (or +/-INF)."""
    if v == INF:
        return 0x7F800000
    if v == -INF:
        return 0xFF800000
    f = float(v)  # exact: binary32 values are binary64 values
    return struct.unpack("<I", struct.pack("<f", f))[0]


# ---- exhaustive code tables, built from the bit-field definitions -------------------


def e2m1_magnitude_value(code: int) -> Fraction:
    e, m = (code >> 1) & 3, code & 1
    if e == 0:
        return Fraction(m, 2)
    return Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))


def e4m3_value(code: int) -> Fraction:
    """Finite non-negative E4M3 values only (codes 0x00..0x7E)."""
    if not 0 <= code <= 0x7E:
        raise ValueError("E4M3 code outside the finite non-negative range")
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return Fraction(m, 512)
    return Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))


E2M1_TABLE = [(c, e2m1_magnitude_value(c)) for c in range(8)]
E4M3_TABLE = [(c, e4m3_value(c)) for c in range(0x7F)]


def nearest_code(v, table) -> int:
    """Brute force: the code whose value is nearest to v >= 0; ties -> even code.

    ``v`` may be +INF, which is nearest to the largest entry (saturation).
    """
    if v == INF:
        return table[-1][0]
    best = None
    for code, val in table:
        dist = abs(val - v)
        if best is None or dist < best[1] or (dist == best[1] and code % 2 == 0):
            best = (code, dist)
    return best[0]


# ---- quantiser ------------------------------------------------------------------------


def quantize_block(xs, gs_bits: int):
    """Quantise one block of 16 values (given as binary32 bit patterns of bf16 values).

    Returns (list of 16 four-bit codes, scale code). Reading R1, exact arithmetic.
    """
    if len(xs) != 16:
        raise ValueError("a block has 16 elements")
    gs = f32_bits_to_fraction(gs_bits)
    vals = [f32_bits_to_fraction(b) for b in xs]
    signs = [(b >> 31) & 1 for b in xs]
    amax = max(abs(v) for v in vals)
    den = rn32(6 * gs)
    s_raw = rn32(amax / den)
    S = nearest_code(s_raw, E4M3_TABLE)
    d = rn32(e4m3_value(S) * gs)
    codes = []
    for v, sg in zip(vals, signs):
        if d == 0:
            mag = 0
        else:
            y = rn32(abs(v) / d)
            mag = nearest_code(y, E2M1_TABLE)
        codes.append((sg << 3) | mag)
    return codes, S


def quantize(rows, gs_bits: int):
    """Quantise a list of rows (each a list of binary32 bit patterns, len % 16 == 0).

    Returns (packed rows as lists of bytes, scale rows as lists of bytes).
    """
    packed, scales = [], []
    for row in rows:
        if len(row) % 16:
            raise ValueError("row length must be a multiple of 16")
        prow, srow = [], []
        for b0 in range(0, len(row), 16):
            codes, S = quantize_block(row[b0:b0 + 16], gs_bits)
            srow.append(S)
            for j in range(8):
                prow.append(codes[2 * j] | (codes[2 * j + 1] << 4))
        packed.append(prow)
        scales.append(srow)
    return packed, scales


def global_scale_bits(amax_bits: int) -> int:
    """RN32(amax / 2688); 1.0 for amax == 0."""
    amax = f32_bits_to_fraction(amax_bits)
    if amax == 0:
        return 0x3F800000
    return fraction_to_f32_bits(rn32(amax / 2688))


def dot_exact(a_codes, a_scales, w_codes, w_scales) -> Fraction:
    """Exact sum_k a_k w_k of two decoded NVFP4 rows (global scales excluded)."""
    a_codes, w_codes = [int(c) for c in a_codes], [int(c) for c in w_codes]
    a_scales, w_scales = [int(c) for c in a_scales], [int(c) for c in w_scales]
    total = Fraction(0)
    for k in range(len(a_codes)):
        qa = e2m1_magnitude_value(a_codes[k] & 7) * (-1 if a_codes[k] & 8 else 1)
        qw = e2m1_magnitude_value(w_codes[k] & 7) * (-1 if w_codes[k] & 8 else 1)
        total += qa * e4m3_value(a_scales[k // 16]) * qw * e4m3_value(w_scales[k // 16])
    return total


def bf16_round_bits(v: Fraction) -> int:
    """bf16 bit pattern of RN(v) with 8 significant bits, ties to even (finite v)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = struct.unpack("<I", struct.pack("<f", float(r)))[0]
    return sign | (f >> 16)
