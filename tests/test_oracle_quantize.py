"""Pins for the oracle's quantiser (CPU only).

Worked blocks below are derived by hand from the format's definition (E2M1 elements,
one E4M3 scale per 16 elements, fp32 global scale: "BFL (fp8r / nvfp4)", nvfp4 item;
zubnet.ai page, paragraph 1) and the R1 operation order stated in the oracle. The
vectorised oracle is further pinned to the exact brute force of
``oracle.scalar_oracle`` and to closed-form invariants.
"""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from oracle import scalar_oracle as S


def f32_to_bf16_bits_exact(vals):
    """bf16 bits of values that are exactly representable in bf16 (asserted)."""
    f = np.asarray(vals, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


# (global scale, 16 values, expected scale byte, expected 8 packed bytes)
WORKED = [
    # A. gs = 2^-6: den = 6/64 = 0.09375; amax 6 -> s_raw = 64 = 2^6 -> E4M3 exponent
    #    field 13, mantissa 0 -> 0x68; d = 64 * 2^-6 = 1, so y = |x|. Codes:
    #    6->7 4->6 3->5 2->4 1.5->3 1->2 .5->1 0->0 -0->8 -6->F; ties: .25->0 .75->2
    #    1.25->2 1.75->4 2.5->4 5->6 (the even code of each pair).
    (2.0**-6, [6, 4, 3, 2, 1.5, 1, 0.5, 0, -0.0, -6, 0.25, 0.75, 1.25, 1.75, 2.5, 5],
     0x68, [0x67, 0x45, 0x23, 0x01, 0xF8, 0x20, 0x42, 0x64]),
    # B. gs = 2^-6, amax 7: s_raw = RN32(7/0.09375) = 74.67 -> nearest E4M3 is 72 =
    #    1.125 * 2^6 -> 0x69; d = 1.125. y: 7->6.22 (7); 1.6875->1.5 (3); 2.8125->2.5
    #    tie (4); .28125->.25 tie (0); .84375->.75 tie (2); -3.9375->3.5 tie (6, neg E);
    #    5.625->5 tie (6); 1.40625->1.25 tie (2); .5625->.5 (1).
    (2.0**-6, [7, 1.6875, 2.8125, 0.28125, 0.84375, -3.9375, 5.625, 1.40625,
               0, 0, 0, 0, 0, 0, 0, 0.5625],
     0x69, [0x37, 0x04, 0xE2, 0x26, 0x00, 0x00, 0x00, 0x10]),
    # C. E4M3-subnormal scale: gs = 1, amax = 41/4096: s_raw = RN32(41/24576) =
    #    0.001668 -> nearest of {0, 2^-9} is 2^-9 -> 0x01; d = 2^-9. y: 41/4096 ->
    #    5.125 (7); 5/1024 -> 2.5 tie (4); -2^-10 -> .5 (1, neg 9).
    (1.0, [41 / 4096, 5 / 1024, -(2.0**-10)] + [0.0] * 13,
     0x01, [0x47, 0x09, 0, 0, 0, 0, 0, 0]),
    # D. static scale too small: gs = 2^-10, amax 10: s_raw = 10/(6*2^-10) = 1706.7
    #    > 448 -> saturate 0x7E; d = 448 * 2^-10 = 0.4375. y: 10 -> 22.9 (7);
    #    2.1875 -> 5 tie (6); 1.09375 -> 2.5 tie (4); -.2734375 -> .625 (1, neg 9).
    (2.0**-10, [10, 2.1875, 1.09375, -0.2734375] + [0.0] * 12,
     0x7E, [0x67, 0x94, 0, 0, 0, 0, 0, 0]),
    # E. zero block with negative zeros: amax 0 -> scale 0 -> d = 0 -> magnitude 0,
    #    sign copied: 0 -> 0x0, -0 -> 0x8.
    (1.0, [0.0, -0.0] * 8, 0x00, [0x80] * 8),
    # F. tiny values under a scale that rounds to 0: amax 2^-100 -> s_raw ~ 2^-102.6
    #    -> 0x00; d = 0; codes keep only the sign: -2^-100 -> 0x8, +2^-100 -> 0x0.
    (1.0, [-(2.0**-100), 2.0**-100] + [0.0] * 14, 0x00, [0x08] + [0] * 7),
]


@pytest.mark.parametrize("case", range(len(WORKED)))
def test_worked_blocks(case):
    gs, vals, want_scale, want_packed = WORKED[case]
    x = f32_to_bf16_bits_exact(vals).reshape(1, 16)
    packed, scales = O.quantize(x, gs)
    assert scales.tolist() == [[want_scale]]
    assert packed.tolist() == [want_packed]
    # the exact brute force agrees as well
    sp, ss = S.quantize([[int(v) << 16 for v in x[0]]], int(np.float32(gs).view(np.uint32)))
    assert ss == [[want_scale]] and sp == [want_packed]


def _brute(x_bits, gs):
    rows = [[int(v) << 16 for v in row] for row in x_bits]
    p, s = S.quantize(rows, int(np.float32(gs).view(np.uint32)))
    return np.array(p, dtype=np.uint8), np.array(s, dtype=np.uint8)


def _random_bf16(rng, shape, kind):
    if kind == "normal":
        v = rng.standard_normal(shape)
    elif kind == "heavy":
        v = rng.standard_t(2.0, size=shape)
    elif kind == "rows":
        v = rng.standard_normal(shape) * np.exp(3 * rng.standard_normal((shape[0], 1)))
    elif kind == "tiny":
        v = rng.standard_normal(shape) * 2.0**-40
    elif kind == "grid":  # values sitting on grid points and midpoints of grid*scale
        g = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6])
        v = rng.choice(g, size=shape) * rng.choice([-1, 1], size=shape)
        v *= 2.0 ** rng.integers(-3, 3, size=(shape[0], 1))
    else:
        raise ValueError(kind)
    from workloads import to_bf16_bits

    return to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("kind", ["normal", "heavy", "rows", "tiny", "grid"])
def test_vectorised_equals_brute_force(kind):
    rng = np.random.default_rng({"normal": 1, "heavy": 2, "rows": 3, "tiny": 4, "grid": 5}[kind])
    x = _random_bf16(rng, (6, 64), kind)
    for gs in [O.global_scale(x), np.float32(O.global_scale(x) * np.float32(0.25)),
               np.float32(1.0 / 3.0), np.float32(2.0**-20)]:
        p, s = O.quantize(x, gs)
        bp, bs = _brute(x, gs)
        assert np.array_equal(s, bs), (kind, gs)
        assert np.array_equal(p, bp), (kind, gs)


def test_r1_operation_order_is_kept():
    """Blocks where reading R1 (round d = s*gs to float32, then round |x|/d to float32,
    then pick the nearest E2M1 value) and the exact-real reading (nearest E2M1 value to
    |x| / (s*gs)) give different codes. The vectorised oracle must agree with the
    exact R1 brute force on every one of them. Cases are built around E2M1 midpoints
    so that the float32 roundings decide."""
    from fractions import Fraction

    rng = np.random.default_rng(77)
    mids = [Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4),
            Fraction(5, 2), Fraction(7, 2), Fraction(5)]
    rows, gss = [], []
    differ = 0
    for _ in range(400):
        s_code = int(rng.integers(0x30, 0x70))
        s_val = S.e4m3_value(s_code)
        t = mids[int(rng.integers(0, len(mids)))]
        xb = int(rng.integers(0x3F80, 0x4000))  # bf16 in [1, 2)
        x = S.f32_bits_to_fraction(xb << 16)
        gs0 = S.rn32(x / (s_val * t))
        gbits = S.fraction_to_f32_bits(gs0) + int(rng.integers(-3, 4))
        gs = S.f32_bits_to_fraction(gbits)
        amax_b = S.bf16_round_bits(6 * s_val * gs)
        row = [amax_b << 16, xb << 16] + [0] * 14
        codes, sc = S.quantize_block(row, gbits)
        if sc != s_code:
            continue
        exact = S.nearest_code(x / (s_val * gs), S.E2M1_TABLE)
        if exact != (codes[1] & 7):
            differ += 1
        rows.append([v >> 16 for v in row])
        gss.append(gbits)
    assert differ > 0, "no block separated R1 from the exact-real reading"
    for row, gbits in zip(rows, gss):
        x = np.array(row, dtype=np.uint16).reshape(1, 16)
        gs = np.uint32(gbits).view(np.float32)
        p, s_ = O.quantize(x, gs)
        bp, bs = _brute(x, gs)
        assert np.array_equal(p, bp) and np.array_equal(s_, bs)


def test_grid_round_trip():
    """With gs = 2^k, a block holding 6*s*gs and every grid value times s*gs encodes
    back to scale s and those exact codes, for every positive E4M3 scale s."""
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for k in (-8, 0, 5):
        gs = np.float32(2.0**k)
        rows = []
        for sc in range(1, 0x7F):
            s = float(O.e4m3_decode(np.array([sc]))[0])
            vals = [6.0] + grid + [-g for g in grid[1:]]
            rows.append([v * s * float(gs) for v in vals])
        x = f32_to_bf16_bits_exact(np.array(rows)).reshape(len(rows), 16)
        p, s = O.quantize(x, gs)
        assert s[:, 0].tolist() == list(range(1, 0x7F))
        codes = O.unpack_codes(p)
        want = [7] + list(range(8)) + [8 | c for c in range(1, 8)]
        assert (codes == np.array(want, dtype=np.uint8)).all()


def _medium_inputs():
    from workloads import make

    out = {}
    for name in ["tiny", "attn_out", "qkv", "batch4_up"]:
        wl = make(name)
        d = wl.generate(with_weights=False) if name != "tiny" else wl.generate()
        out[name] = d["x"][:256]
    return out


def test_block_amax_maps_to_six_and_self_calibrated_max_scale():
    """Block amax encodes as 6 (code 7) whenever its scale is an E4M3 normal, and a
    self-calibrated tensor's largest block scale is exactly 448 (0x7E)."""
    for name, x in _medium_inputs().items():
        gs = O.global_scale(x)
        p, s = O.quantize(x, gs)
        codes = O.unpack_codes(p).reshape(x.shape[0], -1, 16)
        xf = O.bf16_bits_to_f32(x).reshape(x.shape[0], -1, 16)
        arg = np.abs(xf).argmax(axis=-1)
        amax_codes = np.take_along_axis(codes, arg[..., None], axis=-1)[..., 0] & 7
        normal = s >= 0x08
        assert (amax_codes[normal] == 7).all(), name
        assert int(s.max()) == 0x7E or O.tensor_amax(x) == 0, name


def test_global_scale_closed_form():
    x = f32_to_bf16_bits_exact([2688.0, -1.0]).reshape(1, 2)
    assert O.global_scale(x) == np.float32(1.0)
    x = f32_to_bf16_bits_exact([-5376.0, 3.0]).reshape(1, 2)
    assert O.global_scale(x) == np.float32(2.0)
    assert O.global_scale(np.zeros((2, 16), np.uint16)) == np.float32(1.0)
    # RN32(1/2688) as an IEEE float32 division
    x = f32_to_bf16_bits_exact([1.0]).reshape(1, 1)
    assert O.global_scale(x) == np.float32(1.0) / np.float32(2688.0)
    assert S.global_scale_bits(0x3F800000) == int(
        (np.float32(1.0) / np.float32(2688.0)).view(np.uint32))


def test_dequantize_error_bound():
    """Every element is reproduced within half an E2M1 step of its block scale (plus
    the saturation-free guarantee when the scale is normal)."""
    rng = np.random.default_rng(3)
    x = _random_bf16(rng, (32, 256), "normal")
    gs = O.global_scale(x)
    p, s = O.quantize(x, gs)
    xh = O.dequantize(p, s, gs)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    step = (O.e4m3_decode(s) * float(gs))[..., None] * np.ones((1, 1, 16))
    step = step.reshape(32, 256)
    # largest gap between adjacent E2M1 magnitudes is 2 (between 4 and 6), so the error
    # is at most one scale step (reached exactly at the 4|6 midpoint, y = 5).
    assert np.all(np.abs(xh - xf) <= step * (1.0 + 1e-6))


def test_size_identity():
    """NVFP4 storage is 4.5 bits per element (plus 4 bytes per tensor) against bf16's
    16: 16/4.5 = 3.56x, the 'up to 3.5x' memory reduction (zubnet.ai page, ¶2)."""
    M, K = 4608, 3072
    ratio = (2 * M * K) / O.nvfp4_bytes(M, K)
    assert 3.5 < ratio < 16 / 4.5 + 1e-9


def test_input_validation():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 24), np.uint16), 1.0)
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 32), np.uint16), 0.0)
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 32), np.uint16), float("nan"))
    bad = np.zeros((1, 16), np.uint16)
    bad[0, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        O.quantize(bad, 1.0)
