"""nvfp4_gemm_w4a16 (NVFP4 weights, bf16 activations) on the GPU against the oracle.

The reference is the dequantise-only product of "BFL (fp8r / nvfp4)" (text under the
Kernels table): out = w_gs * X @ W_hat^T with X the bf16 activations as they are. As for
the W4A4 GEMM, every output must lie within 2^-10 * sum_k |x_k w_k| + 1 bf16 ulp of the
exact float64 value. Small shapes are compared in full; the FLUX-sized short-activation
workloads run at full size and are compared on sampled rows."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host, u8_to_dev
from oracle import nvfp4_oracle as O
from workloads import make, to_bf16_bits

pytestmark = pytest.mark.gpu


def _run(x, wp, ws, wgs, guard=True):
    M, N = x.shape[0], wp.shape[0]
    if guard:
        out, ok = guarded((M, N), torch.bfloat16)
    else:
        out, ok = torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), (lambda: True)
    nv.gemm_w4a16(bf16_to_dev(x), u8_to_dev(wp), u8_to_dev(ws), float(wgs), out=out)
    return out, ok


def _check(got, x, wp, ws, wgs, label):
    ref, absref = O.w4a16_ref(x, wp, ws, wgs)
    ok, worst, nbad = O.check_gemm(got, ref, absref)
    assert ok, f"{label}: {nbad} elements out of tolerance (worst err/tol {worst:.3g})"


@pytest.mark.parametrize("M,N,K,kernel", [
    # split-K: at most 64 rows, or K % 64 == 32
    (1, 64, 64, "splitk"), (17, 72, 128, "splitk"), (33, 100, 96, "splitk"),
    (64, 3000, 224, "splitk"), (5, 5, 32, "splitk"), (300, 200, 1056, "splitk"),
    (64, 128, 256, "splitk"),
    # at most 16 rows: 4, 8, 12 and 16 weight rows per workgroup, four or eight waves, 1 to
    # 48 groups of 256 along K, ragged last workgroups
    (1, 4, 256, "gemv16"), (5, 101, 256, "gemv16"), (16, 1000, 2816, "gemv16"),
    (3, 2050, 12288, "gemv16"), (1, 3072, 3072, "gemv16"), (16, 3072, 3072, "gemv16"),
    (7, 12285, 512, "gemv16"), (17, 3072, 3072, "gemv16"), (32, 700, 768, "gemv16"),
    (25, 4000, 1280, "gemv16"), (20, 2050, 6144, "gemv16"),
    # the tiles with their waves along N, each ragged in M and N, with one stage (K = 64),
    # a partial last quad of scale stages (K / 64 = 3, 5, 7, 17) and whole quads (10)
    (130, 70, 256, "wide64x128"), (65, 3000, 448, "wide64x128"),
    (1001, 3001, 192, "wide128x128"), (2305, 1537, 128, "wide128x128"),
    (2049, 2081, 64, "wide96x256"), (2300, 2000, 192, "wide96x256"),
    (2017, 2305, 1088, "wide96x256"), (2304, 2048, 640, "wide96x256"),
    (2017, 3000, 320, "wide128x256"),
    (3001, 2999, 192, "wide"), (3300, 2600, 320, "wide"),
    # the 288 x 192 tile (one pass where the others need two) and the 256 x 256 tile, each
    # with one stage and with 17 or 18 (whole quads of scale stages and a partial last one)
    (4288, 3088, 64, "fit"), (4096, 4096, 64, "tile256"),
    (4288, 3088, 1088, "fit"), (4096, 4096, 1152, "tile256"),
])
def test_w4a16_small_shapes_in_full(M, N, K, kernel):
    assert nv.gemm_w4a16_plan(M, N, K) == kernel
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    x = to_bf16_bits((rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wgs = O.global_scale(w)
    wp, ws = O.quantize(w, wgs)
    say("w4a16", M, N, K)
    out, ok = _run(x, wp, ws, wgs)
    got = to_host(out)
    assert ok(), "write outside out"
    _check(got, x, wp, ws, wgs, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,kernel", [
    (17, 4200, 1024, "splitk"), (9, 301, 768, "gemv16"), (20, 130, 512, "gemv16"), (130, 70, 256, "wide64x128"), (2305, 1537, 128, "wide128x128"),
    (2049, 2081, 64, "wide96x256"), (2017, 3000, 320, "wide128x256"), (3001, 2999, 192, "wide"),
    (4288, 3088, 64, "fit"), (4096, 4096, 64, "tile256")])
def test_w4a16_every_scale_code(M, N, K, kernel):
    """Weight scales cycling through all 127 finite E4M3 codes (subnormals and 448
    included) with random codes: pins the scale conversion on every code, in every
    kernel."""
    assert nv.gemm_w4a16_plan(M, N, K) == kernel
    rng = np.random.default_rng(M + N + K)
    x = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = (np.arange(N * (K // 16)) % 127).astype(np.uint8).reshape(N, K // 16)
    ws = ws[rng.permutation(N)]
    wgs = np.float32(2.0**-7)
    say("w4a16 every scale code", M, N, K)
    out, ok = _run(x, wp, ws, wgs)
    got = to_host(out)
    assert ok(), "write outside out"
    _check(got, x, wp, ws, wgs, f"scales {M}x{N}x{K}")


def test_w4a16_identity_weights():
    """W = 3 I under w_gs = 2^-6: every product and sum is exact, out = bf16(3 x)."""
    rng = np.random.default_rng(41)
    K = 128
    x = to_bf16_bits(rng.standard_normal((40, K)).astype(np.float32))
    eye = to_bf16_bits((np.eye(K) * 3.0).astype(np.float32))
    wgs = np.float32(2.0**-6)
    wp, ws = O.quantize(eye, wgs)
    say("w4a16 identity")
    out, _ = _run(x, wp, ws, wgs)
    want = to_bf16_bits(O.bf16_bits_to_f32(x) * np.float32(3.0))
    assert np.array_equal(O.bf16_bits_to_f32(to_host(out)), O.bf16_bits_to_f32(want))


@pytest.mark.parametrize("name", ["odd_m1", "odd_m17", "odd_m256", "tiny"])
def test_w4a16_workloads_full_size_sampled_rows(name):
    wl = make(name)
    d = wl.generate()
    wgs = O.global_scale(d["w"])
    wp, ws = O.quantize(d["w"], wgs)
    say("w4a16 workload", name, wl.M, wl.N, wl.K)
    out, ok = _run(d["x"], wp, ws, wgs)
    got = to_host(out)
    assert ok()
    rows = np.unique(np.array([0, wl.M - 1, wl.M // 2] + list(
        np.random.default_rng(13).choice(wl.M, size=min(32, wl.M), replace=False))))
    _check(got[rows], d["x"][rows], wp, ws, wgs, name)
    out2, _ = _run(d["x"], wp, ws, wgs, guard=False)
    assert np.array_equal(to_host(out2), got)


def test_w4a16_attn_out_shape_sampled_rows():
    """The 4608-token FLUX shape through the same kernel (correctness; the W4A4 GEMM is
    the fast path at this size)."""
    wl = make("attn_out")
    d = wl.generate()
    wgs = O.global_scale(d["w"])
    wp, ws = O.quantize(d["w"], wgs)
    say("w4a16 attn_out")
    out, _ = _run(d["x"], wp, ws, wgs, guard=False)
    got = to_host(out)
    rows = np.array([0, 1, 2303, 4607] + list(np.random.default_rng(14).choice(4608, 12, replace=False)))
    _check(got[rows], d["x"][rows], wp, ws, wgs, "attn_out")


def test_w4a16_binding_rejects_bad_shapes():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros((8, 24), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((8, 3), dtype=torch.uint8, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        nv.gemm_w4a16(x, wp, ws, 1.0)   # K = 48 is not a multiple of 32
