"""Pins for the MXFP8 oracle (CPU only).

MXFP8 per the zubnet.ai page, paragraph 1: OCP microscaling with 8-bit E4M3 elements in
32-element blocks sharing one scale. The scale rule and element rounding are the
readings stated in the oracle's header (shared exponent floor(log2(amax)) - 8, E8M0
byte, E4M3 nearest with ties to even, saturating). Each pin below is checked against
something other than the oracle's own code: closed forms, exact rational brute force,
hand-derived values and error bounds.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import mxfp8_oracle as MX
from oracle import nvfp4_oracle as O
from oracle import scalar_oracle as S
from workloads import to_bf16_bits


def _bits(vals):
    return to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_shared_exponent_closed_forms():
    # 448 = 1.75 * 2^8 -> e = 0; 2^k -> k - 8; just below 2^k -> k - 9
    assert MX.shared_exponent(np.float64([448.0]))[0] == 0
    assert MX.shared_exponent(np.float64([256.0]))[0] == 0
    assert MX.shared_exponent(np.float64([255.0]))[0] == -1
    assert MX.shared_exponent(np.float64([1.0]))[0] == -8
    assert MX.shared_exponent(np.float64([0.99609375]))[0] == -9
    for k in range(-100, 100, 7):
        assert MX.shared_exponent(np.float64([2.0**k]))[0] == k - 8
        assert MX.shared_exponent(np.float64([2.0**k * 1.9921875]))[0] == k - 8
    # all-zero block: byte 0; tiny and huge amax clamp to [-127, 127]
    assert MX.shared_exponent(np.float64([0.0]))[0] == -127
    assert MX.shared_exponent(np.float64([2.0**-133]))[0] == -127
    assert MX.shared_exponent(np.float64([3.3895e38]))[0] == 119


def test_e8m0_decode():
    assert MX.e8m0_decode(np.array([127]))[0] == 1.0
    assert MX.e8m0_decode(np.array([0]))[0] == 2.0**-127
    assert MX.e8m0_decode(np.array([254]))[0] == 2.0**127
    assert np.isnan(MX.e8m0_decode(np.array([255]))[0])


def test_hand_derived_elements():
    """Ties to even, subnormals and saturation, worked by hand. Block of 32 with its
    largest element 448 so the scale is 1 (e = 0) and y = x."""
    vals = np.zeros(32, np.float32)
    vals[0] = 448.0          # sets e = 0
    vals[1] = 1.0625         # tie between 1.0 (0x38) and 1.125 (0x39) -> even 0x38
    vals[2] = 1.1875         # tie between 1.125 (0x39) and 1.25 (0x3A) -> 0x3A
    vals[3] = -1.1875        # sign copied -> 0xBA
    vals[4] = 2.0**-10       # tie between 0 and 2^-9 (code 1) -> 0
    vals[5] = 3 * 2.0**-10   # tie between 2^-9 (1) and 2^-8 (2) -> 2
    vals[6] = -0.0           # -> 0x80
    vals[7] = 248.0          # tie between 240 (0x77) and 256 (0x78) -> even 0x78
    vals[8] = 232.0          # tie between 224 (0x76) and 240 (0x77) -> even 0x76
    vals[9] = 0.001953125    # 2^-9 exactly -> 0x01
    codes, scales = MX.quantize(_bits(vals)[None, :])
    assert scales[0, 0] == 127
    assert list(codes[0, :10]) == [0x7E, 0x38, 0x3A, 0xBA, 0x00, 0x02, 0x80, 0x78, 0x76, 0x01]
    # saturation: amax 464 -> e = 0 and 464 > 448 -> 448 (0x7E), never NaN
    v2 = np.zeros(32, np.float32)
    v2[0] = 464.0
    v2[1] = -500.0
    c2, s2 = MX.quantize(_bits(v2)[None, :])
    assert s2[0, 0] == 127 and c2[0, 0] == 0x7E and c2[0, 1] == 0xFE


def test_on_grid_blocks_round_trip():
    """A block of E4M3 values times 2^e whose largest magnitude lies in [256, 448]
    (E4M3's top binade) quantizes back to exactly those codes and e."""
    rng = np.random.default_rng(7)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    top = np.arange(0x78, 0x7F, dtype=np.uint8)  # 256 .. 448
    rows = []
    want_c, want_s = [], []
    for _ in range(200):
        c = rng.choice(finite, 32)
        c[rng.integers(32)] = rng.choice(top) | (0x80 if rng.integers(2) else 0)
        e = int(rng.integers(-100, 100))
        x = O.e4m3_decode(c) * 2.0**e
        rows.append(x)
        want_c.append(c)
        want_s.append(e + 127)
    codes, scales = MX.quantize(_bits(np.array(rows)))
    assert np.array_equal(codes, np.array(want_c))
    assert np.array_equal(scales[:, 0], np.array(want_s, dtype=np.uint8))


def _scalar_quantize_block(xs):
    """Independent exact-rational MXFP8 quantizer for one block of 32 floats."""
    fr = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        e = -127
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        while Fraction(2) ** e > amax:
            e -= 1
        e = max(-127, min(127, e - 8))
    table = [(c, S.e4m3_value(c)) for c in range(0x7F)]
    codes = []
    for v, xf in zip(fr, xs):
        y = abs(v) / Fraction(2) ** e
        if y >= 448:
            c = 0x7E
        else:
            best = None
            for code, val in table:
                d = abs(val - y)
                if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                    best = (d, code)
            c = best[1]
        if np.signbit(xf):
            c |= 0x80
        codes.append(c)
    return codes, e + 127


def test_brute_force_rationals():
    rng = np.random.default_rng(8)
    blocks = []
    for i in range(60):
        b = rng.standard_normal(32) * np.exp(rng.uniform(-30, 30))
        if i % 5 == 0:
            b[rng.integers(32)] *= 40.0           # one outlier
        if i % 7 == 0:
            b[:8] = 0.0
        blocks.append(b)
    blocks.append(np.zeros(32))
    x = _bits(np.array(blocks))
    codes, scales = MX.quantize(x)
    xf = O.bf16_bits_to_f32(x)
    for r in range(len(blocks)):
        wc, ws = _scalar_quantize_block(xf[r])
        assert list(codes[r]) == wc, r
        assert scales[r, 0] == ws, r


def test_dequantization_error_bound():
    """Unsaturated elements: |x - x_hat| <= half an E4M3 step at |x|'s binade (relative
    2^-4 for normals, absolute 2^-10 * 2^e in the subnormal range); saturated ones lose
    at most |x| - 448 * 2^e."""
    rng = np.random.default_rng(9)
    x = _bits(rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1))))
    codes, scales = MX.quantize(x)
    xf = O.bf16_bits_to_f32(x).astype(np.float64).reshape(64, 8, 32)
    xh = MX.dequantize(codes, scales).reshape(64, 8, 32)
    scale = MX.e8m0_decode(scales)[..., None]
    y = np.abs(xf) / scale
    err = np.abs(xf - xh) / scale
    normal = (y >= 2.0**-6) & (y <= 448)
    assert np.all(err[normal] <= y[normal] * 2.0**-4 * (1 + 1e-12))
    sub = y < 2.0**-6
    assert np.all(err[sub] <= 2.0**-10 * (1 + 1e-12))
    sat = y > 448
    assert np.all(err[sat] <= y[sat] - 448 + 1e-12)


def test_gemm_ref_against_exact_rationals_and_planted_mistakes():
    rng = np.random.default_rng(10)
    M, N, K = 3, 4, 64
    ac, as_ = MX.quantize(_bits(rng.standard_normal((M, K))))
    wc, ws = MX.quantize(_bits(rng.standard_normal((N, K)) * 0.02))
    ref, absref = MX.gemm_ref(ac, as_, wc, ws)

    def val(c, s):
        mag = S.e4m3_value(int(c) & 0x7F)
        return (-mag if int(c) & 0x80 else mag) * Fraction(2) ** (int(s) - 127)

    for m in range(M):
        for n in range(N):
            want = sum(val(ac[m, k], as_[m, k // 32]) * val(wc[n, k], ws[n, k // 32])
                       for k in range(K))
            assert ref[m, n] == float(want)
    out = to_bf16_bits(ref.astype(np.float32))
    assert O.check_gemm(out, ref, absref)[0]
    # planted mistakes: one scale byte off by one, and the weights' rows swapped
    ws2 = ws.copy()
    ws2[0, 0] += 1
    bad, _ = MX.gemm_ref(ac, as_, wc, ws2)
    assert not O.check_gemm(to_bf16_bits(bad.astype(np.float32)), ref, absref)[0]
    bad, _ = MX.gemm_ref(ac, as_, wc[::-1], ws[::-1])
    assert not O.check_gemm(to_bf16_bits(bad.astype(np.float32)), ref, absref)[0]


# ---- E5M2 elements (OCP MXFP8's second element type) --------------------------------


def _e5m2_value(c):
    """Exact value of an E5M2 magnitude code 0..0x7B, from the format's definition."""
    e, m = (c >> 2) & 0x1F, c & 3
    if e == 0:
        return Fraction(m, 4) * Fraction(2) ** -14
    return Fraction(2) ** (e - 15) * (1 + Fraction(m, 4))


def test_e5m2_decode_matches_torch_for_all_bytes():
    import torch

    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = MX.e5m2_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert got[0x7B] == 57344.0 and got[0x7C] == np.inf and got[0x01] == 2.0**-16
    for c in range(0x7C):
        assert got[c] == float(_e5m2_value(c)), c


def test_e5m2_encoder_matches_torch_cast_below_overflow():
    """torch's float8_e5m2 cast rounds to nearest even; it agrees with the oracle's
    encoder wherever it does not overflow (|y| < 61440, the midpoint between the largest
    finite value 57344 and 2^16). Checked on random values over the whole range and on
    every representable value and midpoint, +-3 float32 ulps."""
    import torch

    pos = MX.e5m2_decode(np.arange(0x7C))
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids]).astype(np.float32)
    near = [pts]
    up = dn = pts
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        near += [up, dn]
    rng = np.random.default_rng(31)
    rand = (np.exp2(rng.uniform(-20, 15.9, 200000)) * rng.uniform(1, 2, 200000)).astype(np.float32)
    y = np.concatenate(near + [rand])
    y = y[(y >= 0) & (y < 61440)]
    y = np.concatenate([y, -y])
    want = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = MX.encode_signed(y.astype(np.float64), "e5m2")
    assert np.array_equal(got, want)


def test_e5m2_shared_exponent_closed_forms():
    assert MX.shared_exponent(np.float64([57344.0]), "e5m2")[0] == 0
    assert MX.shared_exponent(np.float64([32768.0]), "e5m2")[0] == 0
    assert MX.shared_exponent(np.float64([32767.0]), "e5m2")[0] == -1
    assert MX.shared_exponent(np.float64([1.0]), "e5m2")[0] == -15
    for k in range(-100, 100, 7):
        assert MX.shared_exponent(np.float64([2.0**k]), "e5m2")[0] == max(k - 15, -127)
        assert MX.shared_exponent(np.float64([2.0**k * 1.9921875]), "e5m2")[0] == max(k - 15, -127)
    assert MX.shared_exponent(np.float64([0.0]), "e5m2")[0] == -127
    assert MX.shared_exponent(np.float64([3.3895e38]), "e5m2")[0] == 112


def test_e5m2_hand_derived_elements():
    """Block whose largest element is 57344, so e = 0 and y = x."""
    vals = np.zeros(32, np.float32)
    vals[0] = 57344.0        # sets e = 0 -> 0x7B
    vals[1] = 1.125          # tie between 1.0 (0x3C) and 1.25 (0x3D) -> even 0x3C
    vals[2] = 1.375          # tie between 1.25 (0x3D) and 1.5 (0x3E) -> 0x3E
    vals[3] = -1.375         # sign copied -> 0xBE
    vals[4] = 2.0**-17       # tie between 0 and 2^-16 (code 1) -> 0
    vals[5] = 3 * 2.0**-17   # tie between 2^-16 (1) and 2^-15 (2) -> 2
    vals[6] = -0.0           # -> 0x80
    vals[7] = 2.0**-16       # exactly the smallest subnormal -> 0x01
    vals[8] = 28672.0        # tie between 24576 (0x76) and 32768 (0x78)? no: 28672 = 0x77
    vals[9] = 30720.0        # tie between 28672 (0x77) and 32768 (0x78) -> even 0x78
    codes, scales = MX.quantize(_bits(vals)[None, :], elem="e5m2")
    assert scales[0, 0] == 127
    assert list(codes[0, :10]) == [0x7B, 0x3C, 0x3E, 0xBE, 0x00, 0x02, 0x80, 0x01, 0x77, 0x78]
    # saturation: amax 60000 -> e = 0 and 60000 > 57344 -> 0x7B, never Inf
    v2 = np.zeros(32, np.float32)
    v2[0] = 60000.0
    v2[1] = -63488.0
    c2, s2 = MX.quantize(_bits(v2)[None, :], elem="e5m2")
    assert s2[0, 0] == 127 and c2[0, 0] == 0x7B and c2[0, 1] == 0xFB


def _scalar_quantize_block_e5m2(xs):
    """Independent exact-rational MXFP8-E5M2 quantizer for one block of 32 floats."""
    fr = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        e = -127
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        while Fraction(2) ** e > amax:
            e -= 1
        e = max(-127, min(127, e - 15))
    table = [(c, _e5m2_value(c)) for c in range(0x7C)]
    codes = []
    for v, xf in zip(fr, xs):
        y = abs(v) / Fraction(2) ** e
        if y >= 57344:
            c = 0x7B
        else:
            best = None
            for code, val in table:
                d = abs(val - y)
                if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                    best = (d, code)
            c = best[1]
        if np.signbit(xf):
            c |= 0x80
        codes.append(c)
    return codes, e + 127


def test_e5m2_brute_force_rationals():
    rng = np.random.default_rng(32)
    blocks = []
    for i in range(60):
        b = rng.standard_normal(32) * np.exp(rng.uniform(-30, 30))
        if i % 5 == 0:
            b[rng.integers(32)] *= 40.0
        if i % 7 == 0:
            b[:8] = 0.0
        if i % 11 == 0:
            b[8:16] *= 2.0**-20          # deep subnormal elements
        blocks.append(b)
    blocks.append(np.zeros(32))
    x = _bits(np.array(blocks))
    codes, scales = MX.quantize(x, elem="e5m2")
    xf = O.bf16_bits_to_f32(x)
    for r in range(len(blocks)):
        wc, ws = _scalar_quantize_block_e5m2(xf[r])
        assert list(codes[r]) == wc, r
        assert scales[r, 0] == ws, r


def test_e5m2_on_grid_blocks_round_trip():
    rng = np.random.default_rng(33)
    finite = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], dtype=np.uint8)
    top = np.arange(0x78, 0x7C, dtype=np.uint8)  # 32768 .. 57344
    rows, want_c, want_s = [], [], []
    for _ in range(200):
        c = rng.choice(finite, 32)
        c[rng.integers(32)] = rng.choice(top) | (0x80 if rng.integers(2) else 0)
        e = int(rng.integers(-90, 90))
        rows.append(np.array([float(_e5m2_value(int(v) & 0x7F)) * (-1 if v & 0x80 else 1)
                              for v in c]) * 2.0**e)
        want_c.append(c)
        want_s.append(e + 127)
    codes, scales = MX.quantize(_bits(np.array(rows)), elem="e5m2")
    assert np.array_equal(codes, np.array(want_c))
    assert np.array_equal(scales[:, 0], np.array(want_s, dtype=np.uint8))


def test_e5m2_dequantization_error_bound():
    """Unsaturated elements: |x - x_hat| <= half an E5M2 step (relative 2^-3 for
    normals, absolute 2^-17 * 2^e in the subnormal range)."""
    rng = np.random.default_rng(34)
    x = _bits(rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1))))
    codes, scales = MX.quantize(x, elem="e5m2")
    xf = O.bf16_bits_to_f32(x).astype(np.float64).reshape(64, 8, 32)
    xh = MX.dequantize(codes, scales, "e5m2").reshape(64, 8, 32)
    scale = MX.e8m0_decode(scales)[..., None]
    y = np.abs(xf) / scale
    err = np.abs(xf - xh) / scale
    normal = (y >= 2.0**-14) & (y <= 57344)
    assert np.all(err[normal] <= y[normal] * 2.0**-3 * (1 + 1e-12))
    sub = y < 2.0**-14
    assert np.all(err[sub] <= 2.0**-17 * (1 + 1e-12))


@pytest.mark.parametrize("a_elem,w_elem", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_gemm_ref_mixed_elements_against_exact_rationals(a_elem, w_elem):
    rng = np.random.default_rng(35)
    M, N, K = 3, 4, 64
    ac, as_ = MX.quantize(_bits(rng.standard_normal((M, K))), elem=a_elem)
    wc, ws = MX.quantize(_bits(rng.standard_normal((N, K)) * 0.02), elem=w_elem)
    ref, absref = MX.gemm_ref(ac, as_, wc, ws, a_elem=a_elem, w_elem=w_elem)

    def val(c, s, elem):
        mag = _e5m2_value(int(c) & 0x7F) if elem == "e5m2" else S.e4m3_value(int(c) & 0x7F)
        return (-mag if int(c) & 0x80 else mag) * Fraction(2) ** (int(s) - 127)

    for m in range(M):
        for n in range(N):
            want = sum(val(ac[m, k], as_[m, k // 32], a_elem) * val(wc[n, k], ws[n, k // 32], w_elem)
                       for k in range(K))
            assert ref[m, n] == float(want)
    # planted mistake: the weights decoded as the other element type
    other = "e4m3" if w_elem == "e5m2" else "e5m2"
    bad, _ = MX.gemm_ref(ac, as_, wc, ws, a_elem=a_elem, w_elem=other)
    assert not O.check_gemm(to_bf16_bits(bad.astype(np.float32)), ref, absref)[0]
