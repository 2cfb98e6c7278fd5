"""GPU self-tests: the exact device functions of the quantize and GEMM kernels, checked
exhaustively or against the CPU oracle."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import say, to_host
from oracle import nvfp4_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    from nvfp4_block_scaled_02_amd import _lib

    return _lib.load_library()


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_e2m1_instruction_equals_software_encoder_on_all_patterns(lib):
    say("e2m1 exhaustive 2^32")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(16, dtype=torch.int32, device="cuda")
    assert lib.nvfp4_selftest_e2m1_exhaustive(_p(cnt), _p(first), _s()) == 0
    n = int(to_host(cnt)[0])
    bad = [hex(v & 0xFFFFFFFF) for v in to_host(first)[: min(n, 16)]]
    assert n == 0, (n, bad)


def test_e2m1_encoders_match_oracle(lib):
    say("e2m1 vs oracle")
    g = np.float32([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6])
    pts = [g]
    up, dn = g, g
    for _ in range(4):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        pts += [up, dn]
    rng = np.random.default_rng(0)
    y = np.concatenate(pts + [rng.uniform(0, 8, 1 << 20).astype(np.float32),
                              np.exp2(rng.uniform(-149, 127, 1 << 18)).astype(np.float32),
                              np.float32([np.inf, 3.4e38, 2.0**-149, 0.0])])
    y = np.concatenate([y, -y])
    yd = torch.from_numpy(y).cuda()
    hw = torch.empty(len(y), dtype=torch.uint8, device="cuda")
    sw = torch.empty_like(hw)
    assert lib.nvfp4_selftest_e2m1_encode(_p(yd), _p(hw), _p(sw), len(y), _s()) == 0
    want = (np.signbit(y).astype(np.uint8) << 3) | O.e2m1_encode_magnitude(np.abs(y))
    assert np.array_equal(to_host(sw), want)
    assert np.array_equal(to_host(hw), want)


def test_division_exhaustive(lib):
    say("division exhaustive")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(16, dtype=torch.int32, device="cuda")
    assert lib.nvfp4_selftest_division(_p(cnt), _p(first), _s()) == 0
    assert int(to_host(cnt)[0]) == 0, [hex(v & 0xFFFFFFFF) for v in to_host(first)]


@pytest.mark.parametrize("gs", [1.0, 2.0**-6, 1.0 / 3.0, 3.7e-4, 2.0**-90, 2.0**90])
def test_block_scale_matches_oracle(lib, gs):
    say("block scale", gs)
    gs = np.float32(gs)
    den = np.float32(np.float32(6.0) * gs)
    pos = O.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    t = (np.concatenate([pos, mids]) * float(den))
    t = t[(t > 0) & (t < 3e38)].astype(np.float32)
    pts = [t]
    up, dn = t, t
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        pts += [up, dn]
    rng = np.random.default_rng(1)
    amax = np.concatenate(pts + [(np.exp2(rng.uniform(-20, 20, 1 << 16)) * float(den)).astype(np.float32),
                                 np.float32([0.0])])
    amax = amax[np.isfinite(amax)]
    amax = (amax.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    ad = torch.from_numpy(amax).cuda()
    code = torch.empty(len(amax), dtype=torch.uint8, device="cuda")
    d = torch.empty(len(amax), dtype=torch.float32, device="cuda")
    assert lib.nvfp4_selftest_block_scale(_p(ad), float(gs), _p(code), _p(d), len(amax), _s()) == 0
    with np.errstate(over="ignore"):
        want = O.e4m3_encode((amax / den).astype(np.float32))
    want_d = (O.e4m3_decode(want).astype(np.float32) * gs).astype(np.float32)
    assert np.array_equal(to_host(code), want)
    assert np.array_equal(to_host(d).view(np.uint32), want_d.view(np.uint32))


def _decode_all(lib):
    nb = 256 * 127 * 4  # each (byte, scale) pair: the byte repeated in a 4-byte group
    byte = np.repeat(np.tile(np.arange(256, dtype=np.uint8), 127), 4)
    scale = np.repeat(np.arange(127, dtype=np.uint8), 256)
    bd = torch.from_numpy(byte).cuda()
    sd = torch.from_numpy(scale).cuda()
    hw = torch.empty(2 * nb, dtype=torch.int16, device="cuda")
    sw = torch.empty_like(hw)
    assert lib.nvfp4_selftest_decode(_p(bd), _p(sd), _p(hw), _p(sw), nb, _s()) == 0
    codes = O.unpack_codes(byte.reshape(1, -1))[0]
    s_el = np.repeat(O.e4m3_decode(scale), 8)
    exact = O.e2m1_decode(codes) * s_el
    want = exact.astype(np.float16)
    assert np.array_equal(want.astype(np.float64), exact)  # q * s is exact in f16
    return codes, np.repeat(scale, 8), want.view(np.uint16), {
        "table": to_host(sw).view(np.uint16), "instruction": to_host(hw).view(np.uint16)}


@pytest.mark.parametrize("path", ["instruction", "table"])
def test_gemm_operand_decode_is_exact(lib, path):
    """Every packed byte under every finite E4M3 scale decodes to q * s exactly (f16)."""
    say("decode all bytes x scales", path)
    codes, scales, want, got_all = _decode_all(lib)
    got = got_all[path]
    bad = np.nonzero(got != want)[0]
    if bad.size:
        value_equal = np.float16(got[bad].view(np.float16)) == np.float16(want[bad].view(np.float16))
        by_scale = np.bincount(scales[bad], minlength=127)
        by_code = np.bincount(codes[bad], minlength=16)
        detail = [(int(i), int(codes[i]), int(scales[i]), hex(int(got[i])), hex(int(want[i])))
                  for i in bad[:12]]
        raise AssertionError(
            f"{path}: {bad.size} mismatches; {int(value_equal.sum())} differ only in the sign "
            f"of zero; by scale code (nonzero) {[(k, int(v)) for k, v in enumerate(by_scale) if v][:40]}; "
            f"by element code {by_code.tolist()}; first {detail}")


def test_bf16_epilogue_conversion_exhaustive(lib):
    """The GEMM epilogues round fp32 to bf16 with gfx950's packed conversion; it must
    equal round-to-nearest-even on the bit pattern for every non-NaN binary32 value
    (subnormals, overflow to infinity and ties included), in both halves."""
    say("bf16 packed conversion exhaustive 2^32")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(16, dtype=torch.int32, device="cuda")
    assert lib.nvfp4_selftest_bf16_exhaustive(_p(cnt), _p(first), _s()) == 0
    n = int(to_host(cnt)[0])
    bad = [hex(v & 0xFFFFFFFF) for v in to_host(first)[: min(n, 16)]]
    assert n == 0, (n, bad)
