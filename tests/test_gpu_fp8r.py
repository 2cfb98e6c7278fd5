"""The rowwise FP8 ("fp8r") path on the GPU against the oracle ("BFL (fp8r / nvfp4)",
fp8r item and Kernels table row; the readings are in the oracle's header).

* Quantization is bit-exact against the oracle (codes and fp32 row scales) on every
  workload (activations and weights) and on adversarial rows: all-zero rows, -0, bf16
  subnormals, huge values, constructed ties, rows whose scale falls below 2^-60 (the
  IEEE-division branch), ragged shapes and K = 16.
* The GEMM lies within 2^-10 * sum |a w| + 1 bf16 ulp of the exact product: small and
  ragged shapes in full, a closed form, FLUX shapes at full size on sampled rows, plus
  determinism.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host, u8_to_dev
from oracle import fp8r_oracle as F
from oracle import nvfp4_oracle as O
from workloads import make, names, to_bf16_bits

pytestmark = pytest.mark.gpu


def _f32_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def _check_quantize(x_bits, label):
    M, K = x_bits.shape
    codes, ok_c = guarded((M, K), torch.uint8)
    scales, ok_s = guarded((M,), torch.float32)
    nv.fp8r_quantize(bf16_to_dev(x_bits), codes=codes, scales=scales)
    wc, ws = F.quantize(x_bits)
    gc, gs = to_host(codes), to_host(scales)
    assert ok_c() and ok_s(), f"{label}: write outside the outputs"
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32)), \
        f"{label}: {np.count_nonzero(gs != ws)} row scales differ"
    assert np.array_equal(gc, wc), f"{label}: {np.count_nonzero(gc != wc)} code bytes differ"


@pytest.mark.parametrize("name", names())
def test_quantize_workloads_bit_exact(name):
    wl = make(name)
    d = wl.generate()
    say("fp8r quantize", name)
    _check_quantize(d["x"], name + "/x")
    _check_quantize(d["w"], name + "/w")


def test_quantize_adversarial():
    rng = np.random.default_rng(61)
    M, K = 29, 784   # ragged rows; K = 98 groups of 8, not a multiple of 64 lanes
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.uniform(-20, 20, (M, 1))).astype(np.float32)
    x[0] = 0.0                                  # all-zero row -> scale 1
    x[1] = -0.0                                 # negative zeros only
    x[2] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0**-128)  # bf16 subnormals
    x[3, :] = np.float32(3.3e38)                # huge
    x[3, 5] = np.float32(-3.3e38)
    x[4] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0**-70)   # s < 2^-60
    x[5] = 0.0                                  # constructed ties with s = 1 (max 448)
    x[5, 0] = 448.0
    x[5, 1:6] = [1.0625, 232.0, 248.0, 3 * 2.0**-10, -1.1875]
    x[6] = rng.standard_normal(K).astype(np.float32) * np.float32(2.0**-52)   # s just above 2^-60
    x[7, :] = 0.0
    x[7, 100] = np.float32(2.0**-133)           # smallest bf16 subnormal as the max
    say("fp8r quantize adversarial")
    _check_quantize(to_bf16_bits(x), "adversarial")


@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (65, 1040), (1000, 3072), (5, 16384), (3, 16400), (9, 24576)])
def test_quantize_shapes(M, K):
    rng = np.random.default_rng(M + K)
    x = to_bf16_bits((rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32))
    say("fp8r quantize", M, K)
    _check_quantize(x, f"{M}x{K}")


def _gemm_dev(ac, as_, wc, ws, guard=True):
    M, N = ac.shape[0], wc.shape[0]
    if guard:
        out, ok = guarded((M, N), torch.bfloat16)
    else:
        out, ok = torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), (lambda: True)
    nv.fp8r_gemm(u8_to_dev(ac), _f32_to_dev(as_), u8_to_dev(wc), _f32_to_dev(ws), out=out)
    return out, ok


@pytest.mark.parametrize("M,N,K", [
    (64, 128, 256), (1, 64, 128), (17, 72, 128), (256, 256, 256), (300, 520, 384),
    (513, 261, 1024), (255, 257, 128), (7, 3, 128), (130, 1030, 640),
    (600, 400, 1152), (289, 193, 640),
    (4096, 4096, 128),   # runs on the 256 x 256 kernel (one pass; the fit tile needs two)
    (4096, 4096, 1152),  # the same kernel over 18 stages
])
def test_gemm_small_shapes_in_full(M, N, K):
    rng = np.random.default_rng(M * 13 + N * 7 + K)
    x = to_bf16_bits((rng.standard_normal((M, K)) * np.exp(rng.uniform(-4, 4, (M, 1)))).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02 * np.exp(rng.uniform(-2, 2, (N, 1)))).astype(np.float32))
    ac, as_ = F.quantize(x)
    wc, ws = F.quantize(w)
    say("fp8r gemm", M, N, K)
    out, ok = _gemm_dev(ac, as_, wc, ws)
    got = to_host(out)
    assert ok(), "write outside out"
    ref, absref = F.gemm_ref(ac, as_, wc, ws)
    good, worst, nbad = O.check_gemm(got, ref, absref)
    assert good, f"{nbad} out of tolerance (worst {worst:.3g})"


def test_gemm_exact_scaling():
    """W = 3 * I: every weight row has amax 3, so its scale is RN32(3/448) and its diagonal
    code is 0x7E (448); each output is the single product s_a * e4m3(a) * 448 * s_w, so it
    is zero exactly where the activation code is zero."""
    rng = np.random.default_rng(62)
    K = 256
    x = to_bf16_bits(rng.standard_normal((70, K)).astype(np.float32))
    ac, as_ = F.quantize(x)
    eye = to_bf16_bits((np.eye(K) * 3.0).astype(np.float32))
    wc, ws = F.quantize(eye)
    assert np.all(wc[np.arange(K), np.arange(K)] == 0x7E)
    say("fp8r gemm identity")
    out, _ = _gemm_dev(ac, as_, wc, ws)
    ref, absref = F.gemm_ref(ac, as_, wc, ws)
    good, worst, nbad = O.check_gemm(to_host(out), ref, absref)
    assert good, f"{nbad} out of tolerance (worst {worst:.3g})"
    got = O.bf16_bits_to_f32(to_host(out))
    assert np.array_equal(got == 0, (ac & 0x7F) == 0)


@pytest.mark.parametrize("name", ["attn_out", "qkv", "mlp_down", "odd_m1000", "tiny", "odd_m17"])
def test_gemm_workloads_sampled_rows(name):
    wl = make(name)
    if wl.K % 128:
        pytest.skip("K % 128 != 0")
    d = wl.generate()
    ac, as_ = F.quantize(d["x"])
    wc, ws = F.quantize(d["w"])
    say("fp8r gemm workload", name)
    out, ok = _gemm_dev(ac, as_, wc, ws, guard=wl.M * wl.N < 64 * 2**20)
    got = to_host(out)
    assert ok()
    rng = np.random.default_rng(63)
    rows = np.unique(np.array([0, wl.M - 1, wl.M // 2] + list(rng.choice(wl.M, size=min(40, wl.M), replace=False))))
    ref, absref = F.gemm_ref(ac[rows], as_[rows], wc, ws)
    good, worst, nbad = O.check_gemm(got[rows], ref, absref)
    assert good, f"{name}: {nbad} out of tolerance (worst {worst:.3g})"
    out2, _ = _gemm_dev(ac, as_, wc, ws, guard=False)
    assert np.array_equal(to_host(out2), got)


def test_binding_rejects_bad_shapes():
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        nv.fp8r_quantize(x, scales=torch.zeros((5,), dtype=torch.float32, device="cuda"))
    c = torch.zeros((4, 96), dtype=torch.uint8, device="cuda")
    s = torch.ones((4,), dtype=torch.float32, device="cuda")
    with pytest.raises(nv.NVFP4Error):   # K % 128 != 0
        nv.fp8r_gemm(c, s, c, s)
