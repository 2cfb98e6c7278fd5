"""Pins for the oracle's GEMM reference and acceptance test (CPU only).

The block-scaled W4A4 product is out[m, n] = a_gs * w_gs * sum_k a[m,k] w[n,k] with
a, w the decoded E2M1 x E4M3 values ("BFL (fp8r / nvfp4)", Kernels table, nvfp4 row:
quantised activations and weights fed to one FP4 GEMM). The float64 reference is pinned
to an exact integer product, to brute force with exact rationals, and to closed forms;
the acceptance test is shown to reject planted mistakes.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from oracle import scalar_oracle as S
from workloads import to_bf16_bits


def _q(rng, rows, K, scale=1.0, kind="normal"):
    if kind == "normal":
        v = rng.standard_normal((rows, K)) * scale
    else:
        v = rng.standard_t(3.0, size=(rows, K)) * scale
    x = to_bf16_bits(v.astype(np.float32))
    gs = O.global_scale(x)
    p, s = O.quantize(x, gs)
    return x, gs, p, s


@pytest.mark.parametrize("M,N,K", [(7, 5, 16), (16, 24, 64), (33, 17, 512)])
def test_float64_reference_equals_exact_integer_product(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    _, ags, ap, as_ = _q(rng, M, K, kind="t")
    _, wgs, wp, ws = _q(rng, N, K, scale=0.02)
    ref, _ = O.gemm_ref(ap, as_, ags, wp, ws, wgs, with_abs=False)
    exact = O.gemm_exact_int(ap, as_, wp, ws).astype(np.float64) * 2.0**-20
    exact *= float(ags) * float(wgs)
    scale = np.abs(exact).max()
    assert np.max(np.abs(ref - exact)) <= 2.0**-40 * scale


def test_k16_brute_force_rationals():
    rng = np.random.default_rng(21)
    _, ags, ap, as_ = _q(rng, 3, 16)
    _, wgs, wp, ws = _q(rng, 4, 16)
    ref, _ = O.gemm_ref(ap, as_, ags, wp, ws, wgs, with_abs=False)
    ac = O.unpack_codes(ap)
    wc = O.unpack_codes(wp)
    g = Fraction(float(ags)) * Fraction(float(wgs))
    for m in range(3):
        for n in range(4):
            want = S.dot_exact(list(ac[m]), list(as_[m]), list(wc[n]), list(ws[n])) * g
            assert ref[m, n] == float(want)


def test_identity_weights_reproduce_dequantised_activations():
    """W = c * I with c on the grid: out = c * w_gs * dequant(A) exactly."""
    rng = np.random.default_rng(4)
    K = 64
    _, ags, ap, as_ = _q(rng, 9, K)
    c = 3.0
    w = to_bf16_bits((np.eye(K) * c).astype(np.float32))
    # static scale 2^-6: s_raw = 3 / (6/64) = 32 (exact E4M3), d = 0.5, 3/0.5 = 6 -> the
    # diagonal quantises to exactly 6 * 32 * 2^-6 = 3
    wgs = np.float32(2.0**-6)
    wp, ws = O.quantize(w, wgs)
    assert np.array_equal(O.dequantize(wp, ws, wgs), np.eye(K) * c)
    ref, _ = O.gemm_ref(ap, as_, ags, wp, ws, wgs, with_abs=False)
    assert np.array_equal(ref, O.dequantize(ap, as_, ags) * c)
    assert np.array_equal(ref, O.dequantize(ap, as_, ags) @ (np.eye(K) * c))


def test_zero_operands_give_zero():
    K = 32
    z = np.zeros((5, K), np.uint16)
    p, s = O.quantize(z, 1.0)
    rng = np.random.default_rng(1)
    _, wgs, wp, ws = _q(rng, 6, K)
    ref, absref = O.gemm_ref(p, s, 1.0, wp, ws, wgs)
    assert np.all(ref == 0) and np.all(absref == 0)
    ok, _, _ = O.check_gemm(np.zeros((5, 6), np.uint16), ref, absref)
    assert ok


def _bf16_of(v):
    return to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_tolerance_accepts_correct_and_rejects_planted_mistakes():
    rng = np.random.default_rng(8)
    M, N, K = 24, 20, 256
    _, ags, ap, as_ = _q(rng, M, K)
    _, wgs, wp, ws = _q(rng, N, K, scale=0.02)
    ref, absref = O.gemm_ref(ap, as_, ags, wp, ws, wgs)
    # a correct answer: the float32 result rounded to bf16
    good = _bf16_of(ref.astype(np.float32))
    assert O.check_gemm(good, ref, absref)[0]
    # a float32 recursive-summation result in the worst order also passes
    A = O.decode_blocks(ap, as_).astype(np.float32)
    W = O.decode_blocks(wp, ws).astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    for k in range(K):
        acc = (acc + np.outer(A[:, k], W[:, k]).astype(np.float32)).astype(np.float32)
    alpha = np.float32(np.float32(ags) * np.float32(wgs))
    assert O.check_gemm(_bf16_of(acc * alpha), ref, absref)[0]
    # planted mistakes: a dropped term, a transposed / shifted operand, a sign error,
    # a missing global scale, a wrong block scale
    dropped = (A[:, 1:].astype(np.float64) @ W[:, 1:].T.astype(np.float64)) * float(alpha)
    assert not O.check_gemm(_bf16_of(dropped), ref, absref)[0]
    shifted = (np.roll(A, 1, axis=1).astype(np.float64) @ W.T.astype(np.float64)) * float(alpha)
    assert not O.check_gemm(_bf16_of(shifted), ref, absref)[0]
    assert not O.check_gemm(_bf16_of(-ref), ref, absref)[0]
    assert not O.check_gemm(_bf16_of(ref / float(wgs)), ref, absref)[0]
    s_bad = as_.copy()
    s_bad[0, 0] += 1
    ref_bad, _ = O.gemm_ref(ap, s_bad, ags, wp, ws, wgs, with_abs=False)
    assert not O.check_gemm(_bf16_of(ref_bad), ref, absref)[0]
    # nibble order swapped within each byte
    swapped = ((ap & 0xF) << 4) | (ap >> 4)
    ref_sw, _ = O.gemm_ref(swapped, as_, ags, wp, ws, wgs, with_abs=False)
    assert not O.check_gemm(_bf16_of(ref_sw), ref, absref)[0]


def test_w4a16_differs_from_w4a4_but_stays_close():
    """Dequantise-only (activations unquantised) output differs slightly from the fused
    W4A4 output ("BFL (fp8r / nvfp4)", text under the Kernels table)."""
    rng = np.random.default_rng(12)
    M, N, K = 16, 16, 512
    x, ags, ap, as_ = _q(rng, M, K)
    _, wgs, wp, ws = _q(rng, N, K, scale=0.02)
    w4a4, absref = O.gemm_ref(ap, as_, ags, wp, ws, wgs)
    w4a16, _ = O.w4a16_ref(x, wp, ws, wgs, with_abs=False)
    diff = np.abs(w4a4 - w4a16)
    assert diff.max() > 0
    # activation quantisation error per element is at most one scale step (6/448 of
    # the block amax relative); bound the output difference by that times |W|.
    X = O.bf16_bits_to_f32(x).astype(np.float64)
    Xh = O.dequantize(ap, as_, ags)
    bound = np.abs(X - Xh) @ np.abs(O.dequantize(wp, ws, wgs)).T
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-30)


def test_w4a16_brute_force_rationals():
    """The W4A16 reference against exact rational arithmetic: each output is
    w_gs * sum_k x_k * e2m1(q_k) * e4m3(s_block) ("BFL (fp8r / nvfp4)", text under the
    Kernels table: weights dequantised, activations left as they are)."""
    rng = np.random.default_rng(31)
    K = 32
    x = to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    _, wgs, wp, ws = _q(rng, 4, K, scale=0.02)
    ref, absref = O.w4a16_ref(x, wp, ws, wgs)
    xf = O.bf16_bits_to_f32(x)
    wc = O.unpack_codes(wp)
    g = Fraction(float(wgs))
    for m in range(3):
        for n in range(4):
            want = Fraction(0)
            want_abs = Fraction(0)
            for k in range(K):
                q = S.e2m1_magnitude_value(int(wc[n, k]) & 7) * (-1 if int(wc[n, k]) & 8 else 1)
                w = q * S.e4m3_value(int(ws[n, k // 16])) * g
                want += Fraction(float(xf[m, k])) * w
                want_abs += abs(Fraction(float(xf[m, k])) * w)
            assert ref[m, n] == float(want)
            assert absref[m, n] == float(want_abs)


def test_w4a16_identity_weights_reproduce_activations():
    """W = c * I with c on the E2M1 grid and w_gs = 2^-6: out = x exactly scaled by c."""
    rng = np.random.default_rng(32)
    K = 64
    x = to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32))
    eye = to_bf16_bits((np.eye(K) * 3.0).astype(np.float32))
    wgs = np.float32(2.0**-6)
    wp, ws = O.quantize(eye, wgs)
    ref, _ = O.w4a16_ref(x, wp, ws, wgs, with_abs=False)
    assert np.array_equal(ref, O.bf16_bits_to_f32(x).astype(np.float64) * 3.0)


def test_w4a16_on_grid_activations_equals_w4a4():
    """Activations that already lie on the NVFP4 grid (dequantised under a power-of-two
    global scale, so they are exact in bf16) give the same product through both paths."""
    rng = np.random.default_rng(33)
    M, N, K = 6, 7, 96
    x0 = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    ags = np.float32(2.0**-4)
    ap, as_ = O.quantize(x0, ags)
    xd = O.dequantize(ap, as_, ags)
    x = to_bf16_bits(xd.astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(x).astype(np.float64), xd)  # exact in bf16
    _, wgs, wp, ws = _q(rng, N, K, scale=0.02)
    w4a4, _ = O.gemm_ref(ap, as_, ags, wp, ws, wgs, with_abs=False)
    w4a16, _ = O.w4a16_ref(x, wp, ws, wgs, with_abs=False)
    assert np.array_equal(w4a4, w4a16)
