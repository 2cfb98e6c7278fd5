"""C-ABI checks that need no GPU: the library loads, exports every function the headers
declare, and rejects bad arguments with the documented status before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from nvfp4_block_scaled_02_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from nvfp4_block_scaled_02_amd import build

        build.build()
    return L.load_library()


def _declared_functions():
    names = set()
    for h in ("nvfp4.h", "nvfp4_selftest.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported_and_bound(lib):
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert declared == set(L.SIGNATURES), declared ^ set(L.SIGNATURES)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == L.ABI_VERSION
    for s in range(8):
        assert lib.nvfp4_status_string(s)
    assert lib.nvfp4_status_string(99) == b"unknown status"


# Fake but aligned device addresses: validation never dereferences them.
P16 = ctypes.c_void_p(0x10000)
P16b = ctypes.c_void_p(0x20000)
NULL = ctypes.c_void_p(0)
ODD = ctypes.c_void_p(0x10008)


def test_quantize_validation(lib):
    q = lib.nvfp4_quantize
    assert q(NULL, 4, 32, 1.0, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, 1.0, NULL, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, 0.0, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, -1.0, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, float("nan"), P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, float("inf"), P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, 2.0**-91, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 32, 2.0**91, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 24, 1.0, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(P16, 4, 0, 1.0, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(P16, -1, 32, 1.0, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(P16, 2**40, 2**40, 1.0, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(ODD, 4, 32, 1.0, P16, P16b, NULL) == L.MISALIGNED
    assert q(P16, 4, 32, 1.0, ODD, P16b, NULL) == L.MISALIGNED
    assert q(P16, 4, 32, 1.0, P16, ctypes.c_void_p(0x20002), NULL) == L.MISALIGNED
    # empty problem: success without touching a device
    assert q(P16, 0, 32, 1.0, P16, P16b, NULL) == L.SUCCESS


def test_gemm_validation(lib):
    g = lib.nvfp4_gemm
    args = [P16, P16b, 1.0, P16, P16b, 1.0, 8, 8, 64, P16, NULL]

    def call(changes):
        a = list(args)
        for k, v in changes.items():
            a[k] = v
        return g(*a)

    assert call({0: NULL}) == L.INVALID_VALUE
    assert call({4: NULL}) == L.INVALID_VALUE
    assert call({9: NULL}) == L.INVALID_VALUE
    assert call({2: 0.0}) == L.INVALID_VALUE
    assert call({5: float("inf")}) == L.INVALID_VALUE
    assert call({8: 40}) == L.INVALID_SHAPE
    assert call({8: 0}) == L.INVALID_SHAPE
    assert call({6: -3}) == L.INVALID_SHAPE
    assert call({7: -3}) == L.INVALID_SHAPE
    assert call({0: ODD}) == L.MISALIGNED
    assert call({9: ODD}) == L.MISALIGNED
    assert call({1: ctypes.c_void_p(0x20001)}) == L.MISALIGNED
    assert call({6: 0}) == L.SUCCESS
    assert call({7: 0}) == L.SUCCESS
    # every pair of valid global scales is accepted, also where their fp32 product is
    # subnormal, zero or infinite (the epilogue applies it as m * 2^e); validation runs
    # before the empty-problem return
    for a_gs, w_gs in ((2.0**-90, 2.0**-90), (2.0**90, 2.0**90), (2.0**-80, 2.0**-70)):
        assert call({2: a_gs, 5: w_gs, 6: 0}) == L.SUCCESS
    assert call({2: 2.0**-91, 6: 0}) == L.INVALID_VALUE


def test_gemm_plan_routes_shapes(lib):
    """The planner (host only) sends the FLUX activations (4608 rows) to the 288 x 192
    tile, at most 32 activation rows with K % 256 == 0 to the 16-row kernel, other short
    activations (at most 32 rows, or a few rows of wide weights) to split-K, a
    few hundred rows whose 64 x 64 tiles fit one pass to the kernel whose waves split K,
    and shapes whose tile count fits 256-tile passes better to the 256 x 256 tile;
    K % 128 != 0 needs the register-staged kernel."""
    def plan(M, N, K, cus=0):
        k = ctypes.c_int(-1)
        st = lib.nvfp4_gemm_plan(M, N, K, cus, ctypes.byref(k))
        return st, k.value

    FIT, TILE, SPLIT, GEN, T128, T128SQ, T12864, WS64, WS128, GEMV = 1, 0, 2, 3, 4, 5, 6, 7, 8, 9
    for M, N, K in [(4608, 3072, 3072), (4608, 12288, 3072), (4608, 3072, 12288),
                    (4608, 9216, 3072), (2600, 3000, 128), (1000, 12288, 3072)]:
        assert plan(M, N, K) == (L.SUCCESS, FIT), (M, N, K)
    # at most 16 rows, or 32 while 16-row workgroups fit one pass (K % 256 == 0): the
    # weights' read spread over the chip
    for M, N, K in [(1, 3072, 3072), (16, 3072, 3072), (17, 3072, 3072), (32, 3072, 3072),
                    (1, 3072, 12288), (5, 12288, 256), (1, 18432, 3072), (16, 18432, 3072),
                    (32, 4096, 3072), (16, 9216, 3072)]:
        assert plan(M, N, K) == (L.SUCCESS, GEMV), (M, N, K)
    assert plan(17, 18432, 3072) == (L.SUCCESS, SPLIT)
    assert plan(32, 4112, 3072) == (L.SUCCESS, SPLIT)
    for M, K in [(1, 3072 + 128), (17, 3072 + 128), (32, 1056)]:   # K % 256 != 0
        assert plan(M, 3072, K) == (L.SUCCESS, SPLIT), (M, K)
    # beyond 32 rows, while its 64 x 64 tiles fit one pass over the compute units, the
    # kernel whose waves split K
    for M in (64, 128, 256, 320):
        assert plan(M, 3072, 3072) == (L.SUCCESS, WS64), M
    for M in (64, 256):
        assert plan(M, 3072, 12288) == (L.SUCCESS, WS64), M
    assert plan(64, 12288, 3072) == (L.SUCCESS, WS64)
    assert plan(256, 3072, 3072, 128) == (L.SUCCESS, T12864)   # two passes on 128 units
    assert plan(256, 3072, 3000) != (L.SUCCESS, WS64)            # K % 512 != 0
    # wide weights with few rows: split-K's workgroups still fill the chip
    assert plan(64, 18432, 3072) == (L.SUCCESS, T128SQ)
    assert plan(128, 12288, 3072) == (L.SUCCESS, T12864)
    assert plan(256, 12288, 3072) == (L.SUCCESS, T128SQ)
    assert plan(512, 12288, 3072) == (L.SUCCESS, T128)
    for M in (1500, 2000):   # a few thousand rows: 128 x 192 tiles
        assert plan(M, 3072, 3072) == (L.SUCCESS, T128), M
    for M in (800, 1000):   # about a thousand rows: 128 x 128 tiles
        assert plan(M, 3072, 3072) == (L.SUCCESS, T128SQ), M
    # ... whose two row bands split K once K is long enough to pay for the reduction
    for K in (6144, 12288):
        assert plan(1000, 3072, K) == (L.SUCCESS, WS128), K
    assert plan(640, 3072, 12288) == (L.SUCCESS, T12864)   # one pass of 128 x 64 tiles
    for M in (384, 512, 600):   # a few hundred rows past one pass of 64 x 64: 128 x 64 tiles
        assert plan(M, 3072, 3072) == (L.SUCCESS, T12864), M
    assert plan(2600, 1650, 128) == (L.SUCCESS, T128)
    assert plan(4096, 4096, 128) == (L.SUCCESS, TILE)
    assert plan(18432, 12288, 3072) == (L.SUCCESS, TILE)
    assert plan(600, 700, 208) == (L.SUCCESS, GEN)   # K % 32 == 16: no split-K either
    assert plan(4608, 3072, 3008) == (L.SUCCESS, GEN)
    # fewer compute units: the same M = 1000 product is worth the larger tiles
    assert plan(1000, 3072, 3072, 32) == (L.SUCCESS, FIT)
    assert plan(8, 8, 40)[0] == L.INVALID_SHAPE
    assert plan(-1, 8, 64)[0] == L.INVALID_SHAPE
    assert lib.nvfp4_gemm_plan(8, 8, 64, 0, None) == L.INVALID_VALUE


def test_gemm_w4a16_plan_routes_shapes(lib):
    """The W4A16 planner (host only): at most 16 rows (or 32 in one pass) with K % 256 == 0
    go to the 16-row kernel, the rest of at most 64 rows (or K % 64 != 0) to split-K;
    longer activations to the tiled kernel with the fewest passes over the compute units
    times its per-stage load cost: the FLUX activations to the 224 x 256 tile with its
    waves along N, medium ones to the smaller tiles along N, and the shapes where 288 x 192
    or 256 x 256 tiles need fewer passes to those."""
    def plan(M, N, K, cus=0):
        k = ctypes.c_int(-1)
        st = lib.nvfp4_gemm_w4a16_plan(M, N, K, cus, ctypes.byref(k))
        return st, k.value

    SPLIT, FIT, TILE, WIDE, W128x256, W96x256, W128x128, W64x128, GEMV = range(9)
    for M, N, K in [(4608, 3072, 3072), (4608, 12288, 3072), (4608, 3072, 12288),
                    (4608, 9216, 3072), (18432, 12288, 3072), (1000, 12288, 3072)]:
        assert plan(M, N, K) == (L.SUCCESS, WIDE), (M, N, K)
    for M, N, K in [(1, 3072, 3072), (16, 3072, 3072), (1, 12288, 3072), (5, 100, 256)]:
        assert plan(M, N, K) == (L.SUCCESS, GEMV), (M, N, K)   # at most 16 rows, K % 256 == 0
    assert plan(8, 18432, 3072) == (L.SUCCESS, SPLIT)          # beyond three passes
    for M in (17, 32):
        assert plan(M, 3072, 3072) == (L.SUCCESS, GEMV), M                 # one pass
    assert plan(17, 4112, 3072) == (L.SUCCESS, SPLIT)
    for M, K in [(33, 3072), (64, 3072), (1, 3136)]:
        assert plan(M, 3072, K) == (L.SUCCESS, SPLIT), (M, K)
    for M in (65, 128, 256, 512):
        assert plan(M, 3072, 3072) == (L.SUCCESS, W64x128), M
    assert plan(1000, 3072, 3072) == (L.SUCCESS, W128x128)
    assert plan(256, 12288, 3072) == (L.SUCCESS, W128x128)
    for M in (1500, 2000):
        assert plan(M, 3072, 3072) == (L.SUCCESS, W96x256), M
    assert plan(2017, 3000, 320) == (L.SUCCESS, W128x256)
    assert plan(4288, 3088, 64) == (L.SUCCESS, FIT)     # 1 pass of 288 x 192, 2 of the others
    assert plan(4096, 4096, 64) == (L.SUCCESS, TILE)    # one pass of 256 x 256 tiles
    assert plan(4608, 3072, 3040) == (L.SUCCESS, SPLIT)  # K % 64 == 32
    assert plan(1000, 3072, 3072, 32) == (L.SUCCESS, WIDE)  # fewer compute units
    assert plan(8, 8, 48)[0] == L.INVALID_SHAPE          # K % 32 != 0
    assert plan(8, 8, 2**22 + 32)[0] == L.INVALID_SHAPE
    assert plan(-1, 8, 64)[0] == L.INVALID_SHAPE
    assert lib.nvfp4_gemm_w4a16_plan(8, 8, 64, 0, None) == L.INVALID_VALUE


def test_linear_plan_fuses_short_activations(lib):
    """nvfp4_linear runs the shortest activations (at most 32 rows, the split-K GEMM's
    one-group shape, and at most 16384 elements, which every workgroup quantizes into its
    LDS) as one kernel; everything else as quantize + GEMM."""
    def plan(M, N, K, cus=0):
        f = ctypes.c_int(-1)
        st = lib.nvfp4_linear_plan(M, N, K, cus, ctypes.byref(f))
        return st, f.value

    for M in (1, 5):
        assert plan(M, 3072, 3072) == (L.SUCCESS, 1), M
    assert plan(1, 64, 32) == (L.SUCCESS, 1)
    assert plan(1, 3072, 12288) == (L.SUCCESS, 1)
    assert plan(32, 3072, 512) == (L.SUCCESS, 1)
    assert plan(32, 3072, 544) == (L.SUCCESS, 0)   # 17408 elements
    # the 16-row kernel's fused form takes up to 24576 elements
    assert plan(2, 96, 12288) == (L.SUCCESS, 1)
    for M in (6, 8):
        assert plan(M, 3072, 3072) == (L.SUCCESS, 1), M
    assert plan(32, 1024, 768) == (L.SUCCESS, 1)
    assert plan(32, 1024, 1024) == (L.SUCCESS, 0)
    for M in (9, 17, 32, 33, 64, 256, 1000, 4608):
        assert plan(M, 3072, 3072) == (L.SUCCESS, 0), M
    assert plan(8, 60, 208) == (L.SUCCESS, 0)     # K % 32 == 16: no split-K
    assert plan(0, 3072, 3072) == (L.SUCCESS, 0)
    assert plan(8, 0, 3072) == (L.SUCCESS, 0)
    assert plan(8, 8, 40)[0] == L.INVALID_SHAPE
    assert lib.nvfp4_linear_plan(8, 8, 64, 0, None) == L.INVALID_VALUE


def test_gemm_w4a16_validation(lib):
    g = lib.nvfp4_gemm_w4a16
    args = [P16, P16b, P16b, 1.0, 8, 8, 64, P16, NULL]

    def call(changes):
        a = list(args)
        for k, v in changes.items():
            a[k] = v
        return g(*a)

    assert call({0: NULL}) == L.INVALID_VALUE
    assert call({1: NULL}) == L.INVALID_VALUE
    assert call({2: NULL}) == L.INVALID_VALUE
    assert call({7: NULL}) == L.INVALID_VALUE
    assert call({3: 0.0}) == L.INVALID_VALUE
    assert call({3: 2.0**91}) == L.INVALID_VALUE
    assert call({6: 48}) == L.INVALID_SHAPE   # K % 32 != 0
    assert call({6: 40}) == L.INVALID_SHAPE
    assert call({6: 2**23}) == L.INVALID_SHAPE
    assert call({4: -1}) == L.INVALID_SHAPE
    assert call({0: ODD}) == L.MISALIGNED
    assert call({1: ODD}) == L.MISALIGNED
    assert call({2: ctypes.c_void_p(0x20002)}) == L.MISALIGNED
    assert call({7: ODD}) == L.MISALIGNED
    assert call({4: 0}) == L.SUCCESS
    assert call({5: 0}) == L.SUCCESS


def test_fp8r_validation(lib):
    q = lib.nvfp4_fp8r_quantize
    assert q(NULL, 4, 64, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 64, NULL, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 64, P16, NULL, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 40, P16, P16b, NULL) == L.INVALID_SHAPE   # K % 16 != 0
    assert q(P16, -1, 64, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(ODD, 4, 64, P16, P16b, NULL) == L.MISALIGNED
    assert q(P16, 4, 64, ODD, P16b, NULL) == L.MISALIGNED
    assert q(P16, 4, 64, P16, ctypes.c_void_p(0x20002), NULL) == L.MISALIGNED
    assert q(P16, 0, 64, P16, P16b, NULL) == L.SUCCESS
    g = lib.nvfp4_fp8r_gemm
    args = [P16, P16b, P16, P16b, 8, 8, 128, P16, NULL]

    def call(changes):
        a = list(args)
        for k, v in changes.items():
            a[k] = v
        return g(*a)

    for k in (0, 1, 2, 3, 7):
        assert call({k: NULL}) == L.INVALID_VALUE
    assert call({6: 64}) == L.INVALID_SHAPE     # K % 128 != 0
    assert call({6: 40}) == L.INVALID_SHAPE
    assert call({4: -1}) == L.INVALID_SHAPE
    assert call({4: 2**24}) == L.INVALID_SHAPE   # (M + 256) * K >= 2^31
    assert call({0: ODD}) == L.MISALIGNED
    assert call({1: ctypes.c_void_p(0x20002)}) == L.MISALIGNED
    assert call({7: ODD}) == L.MISALIGNED
    assert call({4: 0}) == L.SUCCESS
    assert call({5: 0}) == L.SUCCESS


def test_device_scale_validation(lib):
    c = lib.nvfp4_calibrate_device
    assert c(NULL, 64, P16b, NULL) == L.INVALID_VALUE
    assert c(P16, 64, NULL, NULL) == L.INVALID_VALUE
    assert c(P16, -1, P16b, NULL) == L.INVALID_SHAPE
    assert c(ODD, 64, P16b, NULL) == L.MISALIGNED
    assert c(P16, 64, ctypes.c_void_p(0x20002), NULL) == L.MISALIGNED
    q = lib.nvfp4_quantize_devgs
    assert q(P16, 4, 64, NULL, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 40, P16b, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(P16, 4, 64, ctypes.c_void_p(0x20002), P16, P16b, NULL) == L.MISALIGNED
    assert q(P16, 0, 64, P16b, P16, P16b, NULL) == L.SUCCESS
    g = lib.nvfp4_gemm_devgs
    args = [P16, P16b, P16b, P16, P16b, P16b, 8, 8, 64, P16, NULL]

    def call(changes):
        a = list(args)
        for k, v in changes.items():
            a[k] = v
        return g(*a)

    for k in (0, 1, 2, 3, 4, 5, 9):
        assert call({k: NULL}) == L.INVALID_VALUE
    assert call({8: 40}) == L.INVALID_SHAPE
    assert call({2: ctypes.c_void_p(0x20002)}) == L.MISALIGNED
    assert call({6: 0}) == L.SUCCESS
    li = lib.nvfp4_linear_devgs
    assert li(P16, NULL, P16, P16b, P16b, 8, 8, 64, P16, P16, 1 << 20, NULL) == L.INVALID_VALUE
    assert li(P16, P16b, P16, P16b, P16b, 8, 8, 64, P16, P16, 16, NULL) == L.WORKSPACE
    assert li(P16, P16b, P16, P16b, P16b, 0, 8, 64, P16, P16, 1 << 20, NULL) == L.SUCCESS


def test_mxfp8_validation(lib):
    q = lib.nvfp4_mxfp8_quantize
    assert q(NULL, 4, 64, P16, P16b, NULL) == L.INVALID_VALUE
    assert q(P16, 4, 48, P16, P16b, NULL) == L.INVALID_SHAPE   # K % 32 != 0
    assert q(P16, -1, 64, P16, P16b, NULL) == L.INVALID_SHAPE
    assert q(ODD, 4, 64, P16, P16b, NULL) == L.MISALIGNED
    assert q(P16, 4, 64, ODD, P16b, NULL) == L.MISALIGNED
    assert q(P16, 0, 64, P16, P16b, NULL) == L.SUCCESS
    g = lib.nvfp4_mxfp8_gemm
    args = [P16, P16b, P16, P16b, 8, 8, 128, P16, NULL]

    def call(changes):
        a = list(args)
        for k, v in changes.items():
            a[k] = v
        return g(*a)

    assert call({0: NULL}) == L.INVALID_VALUE
    assert call({3: NULL}) == L.INVALID_VALUE
    assert call({6: 64}) == L.INVALID_SHAPE       # K % 128 != 0
    assert call({6: 0}) == L.INVALID_SHAPE
    assert call({4: 2**23, 6: 256}) == L.INVALID_SHAPE  # 32-bit offsets exceeded
    assert call({0: ODD}) == L.MISALIGNED
    assert call({1: ctypes.c_void_p(0x20002)}) == L.MISALIGNED
    assert call({7: ODD}) == L.MISALIGNED
    assert call({4: 0}) == L.SUCCESS
    assert call({5: 0}) == L.SUCCESS


def test_linear_validation_and_workspace(lib):
    ws = lib.nvfp4_linear_workspace_bytes
    assert ws(4608, 3072) == (4608 * 3072 // 2) + ((4608 * 3072 // 16 + 255) // 256 * 256)
    assert ws(3, 16) == 256 + 256
    assert ws(3, 24) == 0 and ws(-1, 16) == 0
    lin = lib.nvfp4_linear
    need = ws(8, 64)
    base = [P16, 1.0, P16b, P16b, 1.0, 8, 8, 64, P16, ctypes.c_void_p(0x40000), need, NULL]
    assert lin(*base[:10], need - 1, NULL) == L.WORKSPACE
    b = list(base)
    b[9] = NULL
    assert lin(*b) == L.INVALID_VALUE
    b = list(base)
    b[0] = ODD
    assert lin(*b) == L.MISALIGNED
    b = list(base)
    b[7] = 72
    assert lin(*b) == L.INVALID_SHAPE
    b = list(base)
    b[5] = 0
    assert lin(*b) == L.SUCCESS


def test_linear_noalloc_validation(lib):
    """The allocation-free linear checks its arguments like nvfp4_linear and refuses a
    problem whose workspace exceeds its 32 MiB static scratch, before any HIP call."""
    lin = lib.nvfp4_linear_noalloc
    ws = lib.nvfp4_linear_workspace_bytes
    base = [P16, 1.0, P16b, P16b, 1.0, 8, 8, 64, P16, NULL]
    b = list(base)
    b[0] = NULL
    assert lin(*b) == L.INVALID_VALUE
    b = list(base)
    b[1] = 0.0
    assert lin(*b) == L.INVALID_VALUE
    b = list(base)
    b[0] = ODD
    assert lin(*b) == L.MISALIGNED
    b = list(base)
    b[7] = 72
    assert lin(*b) == L.INVALID_SHAPE
    b = list(base)
    b[5] = 0
    assert lin(*b) == L.SUCCESS
    # the largest FLUX activations fit; one more row of 12288 does not
    assert ws(4608, 12288) <= 32 << 20 and ws(18432, 3072) <= 32 << 20
    assert ws(4854, 12288) <= 32 << 20 < ws(4855, 12288)
    b = list(base)
    b[5], b[7] = 4855, 12288
    assert lin(*b) == L.TOO_LARGE
    assert lib.nvfp4_status_string(L.TOO_LARGE).startswith(b"problem needs more")


def test_amax_validation(lib):
    out = ctypes.c_void_p(0x30000)
    assert lib.nvfp4_amax(NULL, 16, out, NULL) == L.INVALID_VALUE
    assert lib.nvfp4_amax(P16, -1, out, NULL) == L.INVALID_SHAPE
    assert lib.nvfp4_amax(ODD, 16, out, NULL) == L.MISALIGNED


def test_no_device_is_reported(lib, gpu_available):
    if gpu_available:
        pytest.skip("a GPU is present")
    assert lib.nvfp4_quantize(P16, 4, 32, 1.0, P16, P16b, NULL) == L.UNSUPPORTED_DEVICE
    assert lib.nvfp4_gemm(P16, P16b, 1.0, P16, P16b, 1.0, 8, 8, 64, P16, NULL) == \
        L.UNSUPPORTED_DEVICE
    assert lib.nvfp4_linear_noalloc(P16, 1.0, P16b, P16b, 1.0, 8, 8, 64, P16, NULL) == \
        L.UNSUPPORTED_DEVICE


def test_global_scale_from_amax_matches_oracle(lib):
    from oracle import nvfp4_oracle as O

    rng = np.random.default_rng(0)
    vals = np.concatenate([
        np.float32([0.0, 1.0, 2688.0, 448.0 * 6, 1e-30, 3.3e38]),
        np.exp2(rng.uniform(-120, 120, 5000)).astype(np.float32),
    ])
    for v in vals:
        got = np.float32(lib.nvfp4_global_scale_from_amax(float(v)))
        assert got.view(np.uint32) == O.global_scale_from_amax(v).view(np.uint32), v
    assert np.isnan(lib.nvfp4_global_scale_from_amax(-1.0))
    assert np.isnan(lib.nvfp4_global_scale_from_amax(float("inf")))


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        L.load_library(str(tmp_path / "missing.so"))
