"""Pins for the oracle's element and scale codecs (CPU only).

Each check ties the oracle to something outside itself: the literal E2M1 value set,
PyTorch's float8_e4m3fn conversion (an independent library routine), exact brute force
in ``oracle.scalar_oracle``, or closed-form tie points.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from oracle import scalar_oracle as S

# E2M1 grid of the element format (NVFP4 elements are E2M1; "BFL (fp8r / nvfp4)",
# nvfp4 item; zubnet.ai page, paragraph 1): magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_is_the_grid():
    vals = O.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == GRID
    assert list(vals[8:]) == [-g for g in GRID]
    assert np.signbit(vals[8])  # code 0x8 is negative zero


def test_e2m1_scalar_table_matches():
    assert [float(v) for _, v in S.E2M1_TABLE] == GRID


def test_e4m3_decode_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], theirs[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(theirs[~nan]))


def test_e4m3_extremes():
    assert O.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert O.e4m3_decode(np.array([0x01]))[0] == 2.0**-9
    assert O.e4m3_decode(np.array([0x08]))[0] == 2.0**-6
    assert float(S.e4m3_value(0x7E)) == 448.0


def _torch_e4m3(vals):
    t = torch.from_numpy(np.asarray(vals, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_below_464():
    rng = np.random.default_rng(123)
    # log-uniform over the whole range + values around every code and every midpoint
    v = np.exp2(rng.uniform(-14, np.log2(464.0), 200_000)).astype(np.float32)
    pos = O.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids]).astype(np.float32)
    near = [pts]
    up, dn = pts, pts
    for _ in range(3):  # +-1..3 float32 ulps around every code value and midpoint
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        near += [up, dn]
    extra = np.concatenate(near).astype(np.float32)
    extra = extra[(extra >= 0) & (extra <= 464)]
    allv = np.concatenate([v, extra, np.float32([0.0, 448.0, 464.0])])
    assert np.array_equal(O.e4m3_encode(allv), _torch_e4m3(allv))


def test_e4m3_encode_ties_to_even():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38.
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A): even code 0x3A.
    # 2^-10 lies halfway between 0 and 2^-9: even code 0.
    # 15 * 2^-10 lies halfway between 7*2^-9 (0x07) and 2^-6 (0x08): even code 0x08.
    got = O.e4m3_encode(np.float32([1.0625, 1.1875, 2.0**-10, 15 * 2.0**-10]))
    assert list(got) == [0x38, 0x3A, 0x00, 0x08]


def test_e4m3_encode_saturates():
    v = np.float32([448.0, 449.0, 464.0, 465.0, 480.0, 1e30, np.inf])
    assert list(O.e4m3_encode(v)) == [0x7E] * 7


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(7)
    v = np.exp2(rng.uniform(-12, 10, 3000)).astype(np.float32)
    want = [S.nearest_code(S.f32_bits_to_fraction(int(b)), S.E4M3_TABLE) for b in v.view(np.uint32)]
    assert list(O.e4m3_encode(v)) == want


def test_e2m1_encode_grid_ties_and_saturation():
    g = np.float32(GRID)
    assert list(O.e2m1_encode_magnitude(g)) == list(range(8))
    # midpoints: ties go to the even code (last mantissa bit 0)
    ties = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(O.e2m1_encode_magnitude(ties)) == [0, 2, 2, 4, 4, 6, 6]
    up = np.nextafter(ties, np.float32(np.inf))
    dn = np.nextafter(ties, np.float32(0))
    assert list(O.e2m1_encode_magnitude(up)) == [1, 2, 3, 4, 5, 6, 7]
    assert list(O.e2m1_encode_magnitude(dn)) == [0, 1, 2, 3, 4, 5, 6]
    big = np.float32([6.0, 6.5, 100.0, 3.4e38, np.inf])
    assert list(O.e2m1_encode_magnitude(big)) == [7] * 5


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.uniform(0, 8, 4000), np.exp2(rng.uniform(-30, 3, 1000))]).astype(np.float32)
    want = [S.nearest_code(S.f32_bits_to_fraction(int(b)), S.E2M1_TABLE) for b in y.view(np.uint32)]
    assert list(O.e2m1_encode_magnitude(y)) == want


def test_codecs_reject_nan_and_negative():
    with pytest.raises(ValueError):
        O.e4m3_encode(np.float32([np.nan]))
    with pytest.raises(ValueError):
        O.e2m1_encode_magnitude(np.float32([-1.0]))


def test_rn32_matches_ieee_division_and_product():
    """The scalar oracle's hand-written binary32 rounding equals IEEE float32 ops."""
    rng = np.random.default_rng(5)
    bits_a = rng.integers(0, 0x7F800000, 4000, dtype=np.uint32)
    bits_b = rng.integers(0x00000001, 0x7F800000, 4000, dtype=np.uint32)
    # also bf16-like numerators (short significands) and near-range extremes
    bits_a[:1000] &= np.uint32(0xFFFF0000)
    a = bits_a.view(np.float32)
    b = bits_b.view(np.float32)
    with np.errstate(all="ignore"):
        q = (a / b).astype(np.float32)
        p = (a * b).astype(np.float32)
    for i in range(len(a)):
        fa = S.f32_bits_to_fraction(int(bits_a[i]))
        fb = S.f32_bits_to_fraction(int(bits_b[i]))
        assert S.fraction_to_f32_bits(S.rn32(fa / fb)) == int(q.view(np.uint32)[i]), (a[i], b[i])
        assert S.fraction_to_f32_bits(S.rn32(fa * fb)) == int(p.view(np.uint32)[i]), (a[i], b[i])


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(3000) * np.exp2(rng.uniform(-20, 20, 3000))).astype(np.float32)
    v = np.concatenate([v, np.float32([1.00390625, 1.01171875, -3.0, 0.0])])  # includes ties
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for i, x in enumerate(v):
        got = S.bf16_round_bits(S.f32_bits_to_fraction(int(v.view(np.uint32)[i])))
        if x == 0:
            continue
        assert got == int(want[i]), x


def test_bf16_ulp():
    assert O.bf16_ulp(np.array([1.0]))[0] == 2.0**-7
    assert O.bf16_ulp(np.array([1.99]))[0] == 2.0**-7
    assert O.bf16_ulp(np.array([2.0]))[0] == 2.0**-6
    assert O.bf16_ulp(np.array([-3.0]))[0] == 2.0**-6
    assert O.bf16_ulp(np.array([0.0]))[0] == 2.0**-133
    assert O.bf16_ulp(np.array([2.0**-130]))[0] == 2.0**-133
    # exact powers of two just below/above a binade edge
    assert O.bf16_ulp(np.array([np.nextafter(1024.0, 0)]))[0] == 2.0**2
    assert O.bf16_ulp(np.array([1024.0]))[0] == 2.0**3
