"""Pins for the rowwise FP8 ("fp8r") oracle (CPU only).

fp8r per "BFL (fp8r / nvfp4)", scheme list, fp8r item: E4M3 weights with one fp32 scale
per row, activations quantized to E4M3 per row at run time. The scale rule (amax / 448),
the division and the rounding are the readings stated in the oracle's header. Each pin
ties the oracle to something other than its own code: closed forms, hand-derived codes,
PyTorch's float8_e4m3fn cast (an independent library routine), an exact-rational brute
force with a hand binary32 rounding, error bounds, and exact rational GEMMs.
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import fp8r_oracle as F
from oracle import nvfp4_oracle as O
from oracle import scalar_oracle as S
from workloads import to_bf16_bits


def _bits(vals):
    return to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_row_scale_closed_forms():
    # 448 * 2^k -> 2^k exactly; zero row -> 1
    for k in range(-60, 60, 7):
        assert F.row_scale(np.float32([448.0 * 2.0**k]))[0] == np.float32(2.0**k)
    assert F.row_scale(np.float32([0.0]))[0] == 1.0
    # other maxima: the binary32 nearest to amax / 448, by exact rational rounding
    for a in [1.0, 3.0, 1000.0, 1e-20, 0.0078125 * 3, 65504.0]:
        want = float(S.rn32(Fraction(float(np.float32(a))) / 448))
        assert F.row_scale(np.float32([a]))[0] == np.float32(want), a


def test_hand_derived_codes():
    """A row whose maximum is 448 has scale 1, so y = x. Ties to even, subnormals,
    saturation and -0, worked by hand."""
    vals = np.zeros(32, np.float32)
    vals[0] = 448.0          # sets s = 1 -> 0x7E
    vals[1] = 1.0625         # tie 1.0 (0x38) / 1.125 (0x39) -> even 0x38
    vals[2] = 1.1875         # tie 1.125 (0x39) / 1.25 (0x3A) -> 0x3A
    vals[3] = -1.1875        # sign copied -> 0xBA
    vals[4] = 2.0**-10       # tie 0 / 2^-9 -> 0
    vals[5] = 3 * 2.0**-10   # tie 2^-9 (1) / 2^-8 (2) -> 2
    vals[6] = -0.0           # -> 0x80
    vals[7] = 248.0          # tie 240 (0x77) / 256 (0x78) -> 0x78
    vals[8] = 232.0          # tie 224 (0x76) / 240 (0x77) -> 0x76
    vals[9] = 2.0**-9        # smallest subnormal -> 0x01
    vals[10] = -448.0        # -> 0xFE
    codes, scales = F.quantize(_bits(vals)[None, :])
    assert scales[0] == 1.0
    assert list(codes[0, :11]) == [0x7E, 0x38, 0x3A, 0xBA, 0x00, 0x02, 0x80, 0x78, 0x76, 0x01, 0xFE]
    # a row of zeros (with a -0): scale 1, codes 0 / 0x80
    z = np.zeros(16, np.float32)
    z[3] = -0.0
    c0, s0 = F.quantize(_bits(z)[None, :])
    assert s0[0] == 1.0 and c0[0, 3] == 0x80 and not np.any(np.delete(c0[0], 3))


def test_row_maximum_maps_to_448():
    """Whatever the row, its largest element encodes to +-448 (0x7E / 0xFE): amax / s is
    within one binary32 rounding of 448, which rounds (or clamps) to 448."""
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((200, 96)) * np.exp(rng.uniform(-40, 40, (200, 1))))
    codes, _ = F.quantize(x)
    xf = O.bf16_bits_to_f32(x)
    imax = np.abs(xf).argmax(axis=1)
    got = codes[np.arange(200), imax]
    assert np.all((got & 0x7F) == 0x7E)


def test_on_grid_rows_round_trip():
    """Rows of E4M3 values times 2^k that contain +-448 * 2^k have s = 2^k exactly and
    encode back to exactly their codes (bf16 holds every E4M3 value exactly)."""
    rng = np.random.default_rng(4)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rows, want = [], []
    for _ in range(100):
        c = rng.choice(finite, 64)
        c[rng.integers(64)] = 0x7E | (0x80 if rng.integers(2) else 0)
        k = int(rng.integers(-40, 40))
        rows.append(O.e4m3_decode(c) * 2.0**k)
        want.append((c, 2.0**k))
    codes, scales = F.quantize(_bits(np.array(rows)))
    for r, (c, s) in enumerate(want):
        assert scales[r] == np.float32(s)
        assert np.array_equal(codes[r], c), r


def test_codes_match_torch_float8_cast():
    """The element encoder against PyTorch's float8_e4m3fn conversion (round to nearest
    even) of the same binary32 quotients, which stay within [-448, 448]."""
    rng = np.random.default_rng(5)
    x = _bits(rng.standard_normal((64, 512)) * np.exp(rng.uniform(-10, 10, (64, 1))))
    codes, scales = F.quantize(x)
    xf = O.bf16_bits_to_f32(x)
    y = np.clip(xf / scales[:, None], -448, 448).astype(np.float32)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, theirs)


def _scalar_quantize_row(xs):
    """Independent exact-rational rowwise quantizer: s = RN32(amax / 448) and
    y = RN32(x / s) with the hand binary32 rounding, then the nearest E4M3 by exhaustive
    search (ties to the even code), sign copied."""
    fr = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in fr)
    s = Fraction(1) if amax == 0 else S.rn32(amax / 448)
    out = []
    for v, xf in zip(fr, xs):
        y = abs(S.rn32(v / s))
        y = min(y, Fraction(448))
        c = S.nearest_code(y, S.E4M3_TABLE)
        if np.signbit(xf):
            c |= 0x80
        out.append(c)
    return out, s


def test_brute_force_rationals():
    rng = np.random.default_rng(6)
    rows = []
    for i in range(40):
        r = rng.standard_normal(48) * np.exp(rng.uniform(-30, 30))
        if i % 4 == 0:
            r[rng.integers(48)] *= 300.0       # one outlier: most elements subnormal in E4M3
        if i % 9 == 0:
            r[:10] = 0.0
        rows.append(r)
    rows.append(np.zeros(48))
    x = _bits(np.array(rows))
    codes, scales = F.quantize(x)
    xf = O.bf16_bits_to_f32(x)
    for r in range(len(rows)):
        want, s = _scalar_quantize_row(xf[r])
        assert Fraction(float(scales[r])) == s, r
        assert list(codes[r]) == want, r


def test_division_not_reciprocal_multiplication():
    """Rows where RN32(x / s) and RN32(x * RN32(1/s)) give different codes (found by a
    seeded search): the oracle must follow the division, as the exact-rational brute
    force does."""
    rng = np.random.default_rng(9)
    x = _bits(rng.standard_normal((400, 256)) * np.exp(rng.uniform(-5, 5, (400, 1))))
    xf = O.bf16_bits_to_f32(x)
    amax = np.abs(xf).max(axis=1)
    s = (amax / np.float32(448)).astype(np.float32)
    y_div = np.clip(xf / s[:, None], -448, 448)
    y_mul = np.clip(xf * (np.float32(1) / s)[:, None], -448, 448)
    c_div = F.e4m3_encode_signed(y_div)
    c_mul = F.e4m3_encode_signed(y_mul)
    rows = np.nonzero((c_div != c_mul).any(axis=1))[0][:6]
    assert len(rows) >= 3
    codes, _ = F.quantize(x[rows])
    assert not np.array_equal(codes, c_mul[rows])
    for i, r in enumerate(rows):
        want, _ = _scalar_quantize_row(xf[r])
        assert list(codes[i]) == want, r


def test_dequantization_error_bound():
    """|x - s e4m3(code)| <= s * (half an E4M3 step at |x/s|) + the binary32 rounding of the
    quotient: relative 2^-4 for normal quotients, absolute 2^-10 s below 2^-6."""
    rng = np.random.default_rng(7)
    x = _bits(rng.standard_normal((32, 1024)) * np.exp(rng.uniform(-8, 8, (32, 1))))
    codes, scales = F.quantize(x)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    xh = F.dequantize(codes, scales)
    s = scales.astype(np.float64)[:, None]
    y = np.abs(xf) / s
    err = np.abs(xf - xh) / s
    slack = y * 2.0**-23
    normal = y >= 2.0**-6
    assert np.all(err[normal] <= y[normal] * 2.0**-4 + slack[normal])
    assert np.all(err[~normal] <= 2.0**-10 + slack[~normal])


def test_gemm_ref_against_exact_rationals_and_planted_mistakes():
    rng = np.random.default_rng(8)
    M, N, K = 3, 5, 48
    ac, as_ = F.quantize(_bits(rng.standard_normal((M, K))))
    wc, ws = F.quantize(_bits(rng.standard_normal((N, K)) * 0.02))
    ref, absref = F.gemm_ref(ac, as_, wc, ws)

    def val(c):
        mag = S.e4m3_value(int(c) & 0x7F)
        return -mag if int(c) & 0x80 else mag

    for m in range(M):
        for n in range(N):
            exact = sum(val(ac[m, k]) * val(wc[n, k]) for k in range(K))
            exact *= Fraction(float(as_[m])) * Fraction(float(ws[n]))
            assert abs(Fraction(ref[m, n]) - exact) <= abs(exact) * Fraction(1, 2**50)
    out = to_bf16_bits(ref.astype(np.float32))
    assert O.check_gemm(out, ref, absref)[0]
    # planted mistakes: a weight-row scale doubled, activation scales swapped between rows,
    # and the weight rows reversed
    ws2 = ws.copy()
    ws2[1] *= 2
    bad, _ = F.gemm_ref(ac, as_, wc, ws2)
    assert not O.check_gemm(to_bf16_bits(bad.astype(np.float32)), ref, absref)[0]
    as2 = as_[[1, 0, 2]]
    bad, _ = F.gemm_ref(ac, as2, wc, ws)
    assert not O.check_gemm(to_bf16_bits(bad.astype(np.float32)), ref, absref)[0]
    bad, _ = F.gemm_ref(ac, as_, wc[::-1], ws[::-1])
    assert not O.check_gemm(to_bf16_bits(bad.astype(np.float32)), ref, absref)[0]
