"""nvfp4_gemm and nvfp4_linear on the GPU against the CPU oracle.

The GEMM's exact result has many correct bf16 roundings (summation order is free), so
each output element must lie within 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp of the exact
float64 reference. Shapes here are compared in full; the workloads at full size are in
tests/test_gpu_full_outputs.py."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host, u8_to_dev
from oracle import nvfp4_oracle as O
from workloads import make, names, to_bf16_bits

pytestmark = pytest.mark.gpu


def _operands(x, w, ags=None):
    ags = O.global_scale(x) if ags is None else ags
    wgs = O.global_scale(w)
    ap, as_ = O.quantize(x, ags)
    wp, ws = O.quantize(w, wgs)
    return ags, wgs, ap, as_, wp, ws


def _gemm_dev(ap, as_, ags, wp, ws, wgs, guard=True):
    M, N = ap.shape[0], wp.shape[0]
    if guard:
        out, ok = guarded((M, N), torch.bfloat16)
    else:
        out, ok = torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), (lambda: True)
    nv.gemm(u8_to_dev(ap), u8_to_dev(as_), float(ags), u8_to_dev(wp), u8_to_dev(ws),
            float(wgs), out=out)
    return out, ok


def _assert_close(got_bits, ap, as_, ags, wp, ws, wgs, label):
    ref, absref = O.gemm_ref(ap, as_, ags, wp, ws, wgs)
    ok, worst, nbad = O.check_gemm(got_bits, ref, absref)
    assert ok, f"{label}: {nbad} elements out of tolerance (worst err/tol {worst:.3g})"
    return worst


@pytest.mark.parametrize("M,N,K", [
    (64, 128, 256),      # tiny config shape
    (1, 64, 64), (17, 72, 128), (256, 256, 256), (300, 520, 320), (513, 260, 1024),
    (33, 40, 16), (40, 36, 48), (64, 64, 80), (130, 132, 144),   # K % 64 != 0, K % 32 == 16
    (255, 257, 192), (7, 3, 32),
    # split-K path with a half-filled last 64-element chunk (K % 64 == 32), covering the
    # three workgroup shapes the launcher picks: 32x32, 32x64 and 32x128 outputs
    (5, 200, 96), (100, 70, 224), (3, 5000, 1056), (33, 6144, 96), (256, 12288, 96),
    (640, 3072, 96),
    # few rows, wide weights: split-K over 576 workgroups (more than one pass)
    (1, 18432, 256), (17, 18432, 128),
])
def test_gemm_small_shapes_in_full(M, N, K):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    x = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    ags, wgs, ap, as_, wp, ws = _operands(x, w)
    say("gemm", M, N, K)
    out, ok = _gemm_dev(ap, as_, ags, wp, ws, wgs)
    got = to_host(out)
    assert ok(), "write outside out"
    _assert_close(got, ap, as_, ags, wp, ws, wgs, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,kernel", [
    # 288 x 192 tiles: one stage (K = 128), an odd number of stages, ragged by one row
    # and column, and several scale pairs with an odd count
    (2600, 3000, 128, "fit"), (2900, 3100, 384, "fit"), (2305, 3073, 256, "fit"),
    (2000, 4000, 1152, "fit"),
    # 128 x 192 tiles: the same kinds of cases at a few thousand rows
    (2600, 1650, 384, "tile128"), (2500, 1900, 256, "tile128"), (2000, 2100, 640, "tile128"),
    # 128 x 128 tiles: about a thousand rows
    (1500, 2500, 128, "tile128x128"), (1100, 2200, 384, "tile128x128"),
    (1000, 2900, 640, "tile128x128"),
    # 128 x 64 tiles: a few hundred rows
    (513, 1000, 640, "tile128x64"), (777, 385, 1152, "tile128x64"), (600, 700, 256, "tile128x64"),
    # 64 x 64 tiles whose waves split K: 1 to 7 sets of four stages (each way the last
    # sets are run), ragged rows and columns
    (700, 90, 512, "wsplit64"), (65, 1000, 1024, "wsplit64"), (130, 777, 1536, "wsplit64"),
    (200, 64, 2048, "wsplit64"), (257, 1500, 2560, "wsplit64"), (100, 500, 3072, "wsplit64"),
    (320, 3072, 3584, "wsplit64"),
    # 128 x 128 tiles, two row bands of two waves splitting K: 17, 18 and 21 sets
    (1023, 2049, 4352, "wsplit128"), (1000, 2100, 4608, "wsplit128"), (900, 2600, 5376, "wsplit128"),
    # 256 x 256 tiles: one double stage, and nine (an odd count: the last double stage's
    # second half is the loop's tail)
    (4096, 4096, 128, "tile256"), (4096, 4096, 1152, "tile256"),
    (600, 700, 208, "generic"),
    # at most 32 activation rows: 4, 8, 12 and 16 weight rows per workgroup (one per
    # compute unit at N = 1024, 2048, 3072 and beyond), four or eight waves, one to 48
    # groups of 256 along K (a wave with none, the ring of four refilled), ragged last
    # workgroups, one or two 16-row activation blocks
    (1, 4, 256, "gemv16"), (5, 101, 256, "gemv16"), (16, 1000, 2816, "gemv16"),
    (3, 2050, 12288, "gemv16"), (1, 3072, 3072, "gemv16"), (16, 3072, 3072, "gemv16"),
    (7, 12289, 512, "gemv16"), (2, 5000, 2048, "gemv16"), (17, 3072, 3072, "gemv16"),
    (32, 700, 768, "gemv16"), (25, 4000, 1280, "gemv16"), (20, 2050, 6144, "gemv16"),
])
def test_gemm_tiled_kernels_in_full(M, N, K, kernel):
    assert nv.gemm_plan(M, N, K) == kernel
    rng = np.random.default_rng(M * 17 + N * 3 + K)
    x = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    ags, wgs, ap, as_, wp, ws = _operands(x, w)
    say("gemm", kernel, M, N, K)
    out, ok = _gemm_dev(ap, as_, ags, wp, ws, wgs)
    got = to_host(out)
    assert ok(), "write outside out"
    _assert_close(got, ap, as_, ags, wp, ws, wgs, f"{kernel} {M}x{N}x{K}")


def test_gemm_exact_cases():
    """Closed forms: zero operands give exact zeros; W = 3 * I reproduces the dequantised
    activations (the epilogue rounds them to bf16)."""
    rng = np.random.default_rng(3)
    K = 128
    x = to_bf16_bits(rng.standard_normal((96, K)).astype(np.float32))
    ags = O.global_scale(x)
    ap, as_ = O.quantize(x, ags)
    eye = to_bf16_bits((np.eye(K) * 3.0).astype(np.float32))
    wgs = np.float32(2.0**-6)
    wp, ws = O.quantize(eye, wgs)
    say("gemm identity")
    out, _ = _gemm_dev(ap, as_, ags, wp, ws, wgs)
    want = to_bf16_bits(O.dequantize(ap, as_, ags).astype(np.float32) * np.float32(3.0))
    # alpha = RN(ags * 2^-6) is exact, acc = 3 * 2^6 * q * s is exact, so out is exact
    # (as a value: the sign of a zero output is not part of the contract)
    got = O.bf16_bits_to_f32(to_host(out))
    assert np.array_equal(got, O.bf16_bits_to_f32(want))
    zp, zs = O.quantize(np.zeros((50, K), np.uint16), 1.0)
    out, _ = _gemm_dev(zp, zs, 1.0, wp, ws, wgs)
    assert np.all((to_host(out) & 0x7FFF) == 0)


# Global-scale pairs whose fp32 product leaves the normal binary32 range (each scale is
# valid: in [2^-90, 2^90]). A single fp32 alpha would be subnormal (2 significant bits
# left, 9% off), zero or infinite; the library applies the power of two exactly. Each pair comes
# with block-scale codes that put the outputs in bf16's range: E4M3 0x70..0x7E (128..448)
# for the tiny products, 0x01..0x02 (2^-9, 2^-8) for the huge one.
_EXTREME_PAIRS = [
    (np.float32(1.37 * 2.0**-80), np.float32(2.0**-68), range(0x70, 0x7F)),  # 1.37 * 2^-148
    (np.float32(2.0**-90), np.float32(2.0**-60), range(0x70, 0x7F)),         # 2^-150
    (np.float32(2.0**90), np.float32(1.25 * 2.0**40), range(0x01, 0x03)),    # 1.25 * 2^130
]


@pytest.mark.parametrize("pair", range(len(_EXTREME_PAIRS)))
@pytest.mark.parametrize("M,N,K,kernel", [
    (64, 128, 128, "splitk"), (600, 700, 256, "tile128x64"), (1500, 2500, 128, "tile128x128"),
    (130, 777, 1536, "wsplit64"), (1023, 2049, 4352, "wsplit128"),
    (2600, 1650, 384, "tile128"), (2600, 3000, 128, "fit"), (4096, 4096, 128, "tile256"),
    (600, 700, 208, "generic"), (9, 301, 768, "gemv16"), (20, 130, 512, "gemv16"),
])
def test_gemm_extreme_global_scale_pairs(M, N, K, kernel, pair):
    """Every kernel's epilogue against the oracle (whose a_gs * w_gs is exact in float64)
    for scale pairs whose product is not a normal fp32, with random code bytes; the same
    values passed as device-resident scales give the same bits."""
    assert nv.gemm_plan(M, N, K) == kernel
    ags, wgs, codes = _EXTREME_PAIRS[pair]
    rng = np.random.default_rng(M + N + K + 1000 * pair)
    codes = np.asarray(list(codes), np.uint8)
    ap = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.choice(codes, (M, K // 16))
    ws = rng.choice(codes, (N, K // 16))
    say("gemm extreme scales", kernel, M, N, K, float(ags), float(wgs))
    out, ok = _gemm_dev(ap, as_, ags, wp, ws, wgs)
    got = to_host(out)
    assert ok(), "write outside out"
    ref, absref = O.gemm_ref(ap, as_, ags, wp, ws, wgs)
    assert np.isfinite(ref).all() and np.abs(ref).max() < 2.0**127
    assert np.abs(ref).max() > 2.0**-128            # outputs far above bf16's 2^-133 ulp
    good, worst, nbad = O.check_gemm(got, ref, absref)
    assert good, f"{kernel} {M}x{N}x{K}: {nbad} out of tolerance (worst err/tol {worst:.3g})"
    dev = lambda v: torch.tensor([float(v)], dtype=torch.float32, device="cuda")
    o2 = nv.gemm(u8_to_dev(ap), u8_to_dev(as_), dev(ags), u8_to_dev(wp), u8_to_dev(ws), dev(wgs))
    assert np.array_equal(to_host(o2), got)


def _sample_rows(M, rng, n=48):
    rows = {0, M - 1, M // 2}
    rows |= set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["tiny", "attn_out", "mlp_up_static", "odd_m17", "odd_m256", "odd_m1000"])
def test_linear_matches_quantize_then_gemm(name):
    wl = make(name)
    d = wl.generate()
    ags = O.global_scale(d.get("calib", d["x"]))
    wgs = O.global_scale(d["w"])
    wp, ws = O.quantize(d["w"], wgs)
    xd = bf16_to_dev(d["x"])
    ws_bytes = nv.linear_workspace_bytes(wl.M, wl.K)
    work = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    say("linear", name)
    out = nv.linear(xd, float(ags), u8_to_dev(wp), u8_to_dev(ws), float(wgs), workspace=work)
    got = to_host(out)
    qp, qs = nv.workspace_views(work, wl.M, wl.K)
    ap, as_ = O.quantize(d["x"], ags)
    assert np.array_equal(to_host(qp), ap) and np.array_equal(to_host(qs), as_)
    g2, _ = _gemm_dev(ap, as_, ags, wp, ws, wgs, guard=False)
    assert np.array_equal(to_host(g2), got)
    rows = _sample_rows(wl.M, np.random.default_rng(12), n=32)
    _assert_close(got[rows], ap[rows], as_[rows], ags, wp, ws, wgs, name)


@pytest.mark.parametrize("M,N,K,plan", [(1, 640, 256, "fused"), (17, 3072, 1024, "fused"),
                                         (16, 3072, 1280, "fused"), (32, 3072, 2304, "two_kernels"),
                                         (17, 3072, 1056, "two_kernels"),
                                         (600, 700, 256, "two_kernels")])
def test_linear_calibrated_scales_with_subnormal_product(M, N, K, plan):
    """nvfp4_linear on tensors of magnitude 2^-70 and 2^-60 (all positive, so the sums do
    not cancel): their calibrated global scales multiply to about 2^-149, below fp32's
    normal range, while the outputs (about 2^-122) are normal bf16. Workspace bit-exact,
    output within tolerance, and equal to quantize-then-GEMM."""
    assert nv.linear_plan(M, N, K) == plan
    rng = np.random.default_rng(M + N + K)
    x = to_bf16_bits((np.abs(rng.standard_normal((M, K))) * 2.0**-70).astype(np.float32))
    w = to_bf16_bits((np.abs(rng.standard_normal((N, K))) * 2.0**-60).astype(np.float32))
    ags, wgs = O.global_scale(x), O.global_scale(w)
    assert float(np.float32(ags) * np.float32(wgs)) < 2.0**-126
    wp, ws = O.quantize(w, wgs)
    work = torch.empty(nv.linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    say("linear subnormal scale product", M, N, K)
    out = nv.linear(bf16_to_dev(x), float(ags), u8_to_dev(wp), u8_to_dev(ws), float(wgs),
                    workspace=work)
    got = to_host(out)
    qp, qs = nv.workspace_views(work, M, K)
    ap, as_ = O.quantize(x, ags)
    assert np.array_equal(to_host(qp), ap) and np.array_equal(to_host(qs), as_)
    ref, absref = O.gemm_ref(ap, as_, ags, wp, ws, wgs)
    assert np.abs(ref).min() > 2.0**-126
    good, worst, nbad = O.check_gemm(got, ref, absref)
    assert good, f"{nbad} out of tolerance (worst err/tol {worst:.3g})"
    g2, _ = _gemm_dev(ap, as_, ags, wp, ws, wgs, guard=False)
    assert np.array_equal(to_host(g2), got)


def test_operands_beyond_32bit_offsets():
    """Largest-size case: 4 194 081 activation rows x K = 1024, so the packed activations
    (2.1 GB) pass 2^31 bytes and the bf16 input (8.6 GB) passes 2^32; the planner sends
    the GEMM to the register-staged kernel (64-bit addressing). Generated on the device;
    rows straddling the 2^31- and 2^32-byte boundaries of either tensor, and the ends, are
    checked against the oracle: quantization bit-exact, GEMM within the bound."""
    M, N, K = (1 << 22) + 777, 72, 1024
    assert nv.gemm_plan(M, N, K) == "generic"
    gen = torch.Generator(device="cuda").manual_seed(21)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, 1 << 20):   # fp32 draws in slices, rounded to bf16
        r1 = min(M, r0 + (1 << 20))
        x[r0:r1] = torch.randn((r1 - r0, K), device="cuda", generator=gen).to(torch.bfloat16)
    rng = np.random.default_rng(22)
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    ags = nv.calibrate(x)
    wgs = O.global_scale(w)
    wp, ws = O.quantize(w, wgs)
    say("gemm beyond 32-bit offsets", M, N, K)
    ap, as_ = nv.quantize(x, ags)
    out = nv.gemm(ap, as_, ags, u8_to_dev(wp), u8_to_dev(ws), float(wgs))
    torch.cuda.synchronize()
    rows = sorted({0, 1, M - 1, M - 2, M // 2,
                   (1 << 22) - 1, 1 << 22, (1 << 22) + 1,     # packed rows across 2^31 bytes
                   (1 << 20) - 1, 1 << 20, (1 << 21) - 1, 1 << 21,  # bf16 rows across 2^31, 2^32
                   *rng.choice(M, 24, replace=False).tolist()})
    idx = torch.tensor(rows, device="cuda")
    xs = x.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    want_p, want_s = O.quantize(xs, np.float32(ags))
    got_p = ap.index_select(0, idx).cpu().numpy()
    got_s = as_.index_select(0, idx).cpu().numpy()
    assert np.array_equal(got_p, want_p) and np.array_equal(got_s, want_s)
    got = out.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    _assert_close(got, want_p, want_s, ags, wp, ws, wgs, "beyond 32-bit offsets")
    del x, ap, as_, out
    torch.cuda.empty_cache()
