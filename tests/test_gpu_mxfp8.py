"""The MXFP8 path on the GPU against the oracle (OCP microscaling, zubnet.ai page,
paragraph 1; the readings are in the oracle's header).

* The gfx950 fp8 conversion equals the software E4M3 encoder on every binary32 pattern
  (clamped to +-448 as the quantizer does).
* Quantization is bit-exact against the oracle on every workload (activations and
  weights) and on adversarial tensors (zero blocks, -0, bf16 subnormals, huge values,
  constructed ties, ragged shapes).
* The GEMM lies within 2^-10 * sum |a w| + 1 bf16 ulp of the exact float64 product:
  small shapes in full, FLUX shapes at full size on sampled rows, plus determinism.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host, u8_to_dev
from oracle import mxfp8_oracle as MX
from oracle import nvfp4_oracle as O
from workloads import make, names, to_bf16_bits

pytestmark = pytest.mark.gpu


def test_e4m3_conversion_exhaustive():
    lib = nv.load_library()
    count = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(16, dtype=torch.int32, device="cuda")
    say("mxfp8 e4m3 exhaustive")
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.nvfp4_selftest_mxfp8_e4m3_exhaustive(
        ctypes.c_void_p(count.data_ptr()), ctypes.c_void_p(first.data_ptr()), st) == 0
    n = int(to_host(count)[0])
    assert n == 0, f"{n} mismatches, first {[hex(int(v) & 0xFFFFFFFF) for v in to_host(first)[:min(n, 16)]]}"


def _check_quantize(x_bits, label):
    codes, scales = nv.mxfp8_quantize(bf16_to_dev(x_bits))
    wc, ws = MX.quantize(x_bits)
    gc, gs = to_host(codes), to_host(scales)
    assert np.array_equal(gs, ws), f"{label}: {np.count_nonzero(gs != ws)} scale bytes differ"
    assert np.array_equal(gc, wc), f"{label}: {np.count_nonzero(gc != wc)} code bytes differ"


@pytest.mark.parametrize("name", names())
def test_quantize_workloads_bit_exact(name):
    wl = make(name)
    if wl.K % 32:
        pytest.skip("K % 32 != 0")
    d = wl.generate()
    say("mxfp8 quantize", name)
    _check_quantize(d["x"], name + "/x")
    _check_quantize(d["w"], name + "/w")


def test_quantize_adversarial():
    rng = np.random.default_rng(51)
    M, K = 37, 544   # ragged rows, K = 17 blocks
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.uniform(-20, 20, (M, 1))).astype(np.float32)
    x[0, :64] = 0.0                       # zero blocks
    x[1, :32] = -0.0                      # negative zeros only
    x[2, :32] = np.float32(2.0**-133)     # bf16 subnormal amax -> clamped exponent
    x[3, :32] = np.float32(3.3e38)        # huge
    x[4, :32] = np.float32(-3.3e38)
    # constructed ties at e = 0 (block max 448): 1.0625, 232, 248, 3 * 2^-10
    x[5, :32] = 0.0
    x[5, 0] = 448.0
    x[5, 1:5] = [1.0625, 232.0, 248.0, 3 * 2.0**-10]
    x[6, :32] = rng.standard_normal(32).astype(np.float32) * 2.0**-130  # all subnormal-ish
    xb = to_bf16_bits(x)
    say("mxfp8 quantize adversarial")
    _check_quantize(xb, "adversarial")


def _gemm_dev(ac, as_, wc, ws, guard=True):
    M, N = ac.shape[0], wc.shape[0]
    if guard:
        out, ok = guarded((M, N), torch.bfloat16)
    else:
        out, ok = torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), (lambda: True)
    nv.mxfp8_gemm(u8_to_dev(ac), u8_to_dev(as_), u8_to_dev(wc), u8_to_dev(ws), out=out)
    return out, ok


@pytest.mark.parametrize("M,N,K", [
    (64, 128, 256), (1, 64, 128), (17, 72, 128), (256, 256, 256), (300, 520, 384),
    (513, 260, 1024), (255, 257, 128), (7, 3, 128),
    # 288 x 192 tiles with ragged edges and several 8-stage scale groups (K = 1152)
    (600, 400, 1152), (289, 193, 640),
    # 4096 x 4096: 256 x 256 tiles need one pass over 256 compute units, 288 x 192 two,
    # so these run on the 256 x 256 kernel: two stages, and 18 (two whole 8-stage scale
    # groups and a partial third)
    (4096, 4096, 128), (4096, 4096, 1152),
])
def test_gemm_small_shapes_in_full(M, N, K):
    rng = np.random.default_rng(M * 11 + N * 5 + K)
    x = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    ac, as_ = MX.quantize(x)
    wc, ws = MX.quantize(w)
    say("mxfp8 gemm", M, N, K)
    out, ok = _gemm_dev(ac, as_, wc, ws)
    got = to_host(out)
    assert ok(), "write outside out"
    ref, absref = MX.gemm_ref(ac, as_, wc, ws)
    good, worst, nbad = O.check_gemm(got, ref, absref)
    assert good, f"{nbad} out of tolerance (worst {worst:.3g})"


def test_gemm_exact_scaling():
    """W = c * I (c on the E4M3 grid): out = c * dequant(A), every product exact and each
    output a single product, so out is bf16(c * a) exactly."""
    rng = np.random.default_rng(52)
    K = 256
    x = to_bf16_bits(rng.standard_normal((70, K)).astype(np.float32))
    ac, as_ = MX.quantize(x)
    eye = to_bf16_bits((np.eye(K) * 3.0).astype(np.float32))
    wc, ws = MX.quantize(eye)
    say("mxfp8 gemm identity")
    out, _ = _gemm_dev(ac, as_, wc, ws)
    want = to_bf16_bits((MX.dequantize(ac, as_) * 3.0).astype(np.float32))
    assert np.array_equal(O.bf16_bits_to_f32(to_host(out)), O.bf16_bits_to_f32(want))


@pytest.mark.parametrize("name", ["attn_out", "qkv", "mlp_down", "odd_m1000", "tiny"])
def test_gemm_workloads_sampled_rows(name):
    wl = make(name)
    if wl.K % 128:
        pytest.skip("K % 128 != 0")
    d = wl.generate()
    ac, as_ = MX.quantize(d["x"])
    wc, ws = MX.quantize(d["w"])
    say("mxfp8 gemm workload", name)
    out, ok = _gemm_dev(ac, as_, wc, ws, guard=wl.M * wl.N < 64 * 2**20)
    got = to_host(out)
    assert ok()
    rng = np.random.default_rng(53)
    rows = np.unique(np.array([0, wl.M - 1, wl.M // 2] + list(rng.choice(wl.M, size=min(40, wl.M), replace=False))))
    ref, absref = MX.gemm_ref(ac[rows], as_[rows], wc, ws)
    good, worst, nbad = O.check_gemm(got[rows], ref, absref)
    assert good, f"{name}: {nbad} out of tolerance (worst {worst:.3g})"
    out2, _ = _gemm_dev(ac, as_, wc, ws, guard=False)
    assert np.array_equal(to_host(out2), got)


# ---- E5M2 elements ------------------------------------------------------------------


def test_e5m2_conversion_exhaustive():
    """gfx950's bf8 conversion equals the software E5M2 encoder on every binary32 pattern
    (clamped to +-57344 as the quantizer does)."""
    import ctypes

    lib = nv.load_library()
    count = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(16, dtype=torch.int32, device="cuda")
    say("mxfp8 e5m2 exhaustive")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.nvfp4_selftest_mxfp8_e5m2_exhaustive(
        ctypes.c_void_p(count.data_ptr()), ctypes.c_void_p(first.data_ptr()), st) == 0
    n = int(to_host(count)[0])
    assert n == 0, f"{n} mismatches, first {[hex(int(v) & 0xFFFFFFFF) for v in to_host(first)[:min(n, 16)]]}"


def _check_quantize_e5m2(x_bits, label):
    codes, scales = nv.mxfp8_quantize(bf16_to_dev(x_bits), elem="e5m2")
    wc, ws = MX.quantize(x_bits, elem="e5m2")
    gc, gs = to_host(codes), to_host(scales)
    assert np.array_equal(gs, ws), f"{label}: {np.count_nonzero(gs != ws)} scale bytes differ"
    assert np.array_equal(gc, wc), f"{label}: {np.count_nonzero(gc != wc)} code bytes differ"


@pytest.mark.parametrize("name", ["tiny", "attn_out", "qkv", "mlp_down", "odd_m1", "odd_m1000"])
def test_quantize_e5m2_workloads_bit_exact(name):
    wl = make(name)
    d = wl.generate()
    say("mxfp8 e5m2 quantize", name)
    _check_quantize_e5m2(d["x"], name + "/x")
    _check_quantize_e5m2(d["w"], name + "/w")


def test_quantize_e5m2_adversarial():
    rng = np.random.default_rng(61)
    M, K = 37, 544
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.uniform(-20, 20, (M, 1))).astype(np.float32)
    x[0, :64] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = np.float32(2.0**-133)     # bf16 subnormal amax -> clamped exponent
    x[3, :32] = np.float32(3.3e38)
    x[4, :32] = np.float32(-3.3e38)
    # ties at e = 0 (block max 57344): 1.125, 1.375, 3 * 2^-17, 30720
    x[5, :32] = 0.0
    x[5, 0] = 57344.0
    x[5, 1:5] = [1.125, 1.375, 3 * 2.0**-17, 30720.0]
    x[6, :32] = rng.standard_normal(32).astype(np.float32) * 2.0**-130
    x[7, :32] = 0.0
    x[7, 0] = 61000.0                     # e = 0, saturates to 57344
    x[7, 1] = -60000.0
    xb = to_bf16_bits(x)
    say("mxfp8 e5m2 quantize adversarial")
    _check_quantize_e5m2(xb, "adversarial")


@pytest.mark.parametrize("a_elem,w_elem", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("M,N,K", [(64, 128, 256), (17, 72, 128), (300, 520, 384), (600, 400, 1152),
                                   (289, 193, 640), (4096, 4096, 128)])
def test_gemm_mixed_elements_in_full(a_elem, w_elem, M, N, K):
    """Each operand's element type reaches the MFMA's operand format: every output within
    the bound, on the 288 x 192 and 256 x 256 kernels (4096 x 4096 takes the latter)."""
    rng = np.random.default_rng(M * 13 + N * 3 + K)
    x = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    ac, as_ = MX.quantize(x, elem=a_elem)
    wc, ws = MX.quantize(w, elem=w_elem)
    say("mxfp8 gemm", a_elem, w_elem, M, N, K)
    out, ok = guarded((M, N), torch.bfloat16)
    nv.mxfp8_gemm(u8_to_dev(ac), u8_to_dev(as_), u8_to_dev(wc), u8_to_dev(ws), out=out,
                  a_elem=a_elem, w_elem=w_elem)
    got = to_host(out)
    assert ok(), "write outside out"
    ref, absref = MX.gemm_ref(ac, as_, wc, ws, a_elem=a_elem, w_elem=w_elem)
    good, worst, nbad = O.check_gemm(got, ref, absref)
    assert good, f"{nbad} out of tolerance (worst {worst:.3g})"


def test_element_type_is_validated():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        nv.mxfp8_quantize(x, elem="e3m4")
    import ctypes

    lib = nv.load_library()
    c = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    assert lib.nvfp4_mxfp8_quantize_elem(P(x), 4, 64, 2, P(c), P(s), None) == 1
