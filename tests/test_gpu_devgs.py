"""Device-resident global scales on the GPU: calibration on the device equals the
oracle's global scale (the pages' calibrated fp32 input_scale, "BFL (fp8r / nvfp4)",
nvfp4 item), and the quantize, GEMM and linear calls that read their global scales from
device memory are bit-identical to the calls that take them as arguments.

The clamp of a device scale into [2^-90, 2^90] (and NaN or <= 0 read as 1) is a
convention of this library: a device value cannot be validated before launch, and the
quantizer's divisions are exact inside that range. Its cases are closed forms.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, say, to_host, u8_to_dev
from oracle import nvfp4_oracle as O
from workloads import make, to_bf16_bits

pytestmark = pytest.mark.gpu


def _dev_scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _f32_bits(v):
    return np.float32(v).view(np.uint32)


@pytest.mark.parametrize("name", ["tiny", "attn_out", "mlp_up_static", "qkv", "odd_m17"])
def test_calibrate_device_matches_oracle(name):
    d = make(name).generate()
    for key in ("x", "w"):
        say("calibrate_device", name, key)
        got = to_host(nv.calibrate_device(bf16_to_dev(d[key])))[0]
        want = O.global_scale(d[key])
        assert _f32_bits(got) == _f32_bits(want), (key, got, want)
        # the host formula on the device amax gives the same value
        assert _f32_bits(got) == _f32_bits(nv.calibrate(bf16_to_dev(d[key])))


def test_calibrate_device_closed_forms():
    z = torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda")
    assert to_host(nv.calibrate_device(z))[0] == 1.0
    tiny = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    tiny[1, 7] = 2.0**-100            # RN(2^-100 / 2688) < 2^-90: clamped
    assert to_host(nv.calibrate_device(tiny))[0] == np.float32(2.0**-90)
    huge = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    huge[0, 3] = -(2.0**110)          # RN(2^110 / 2688) > 2^90: clamped
    assert to_host(nv.calibrate_device(huge))[0] == np.float32(2.0**90)
    edge = torch.zeros((1, 16), dtype=torch.bfloat16, device="cuda")
    edge[0, 0] = 2688.0               # exactly 1
    assert to_host(nv.calibrate_device(edge))[0] == 1.0


@pytest.mark.parametrize("gs_dev,gs_host", [
    (None, None),                       # the oracle's global scale of x
    (2.0**100, 2.0**90), (2.0**-120, 2.0**-90),
    (float("nan"), 1.0), (-3.0, 1.0), (0.0, 1.0),
])
def test_quantize_devgs_bit_exact(gs_dev, gs_host):
    rng = np.random.default_rng(71)
    x = to_bf16_bits((rng.standard_normal((130, 512)) * np.exp(rng.uniform(-6, 6, (130, 1)))).astype(np.float32))
    if gs_dev is None:
        gs_dev = gs_host = float(O.global_scale(x))
    say("quantize_devgs", gs_dev)
    xd = bf16_to_dev(x)
    p1, s1 = nv.quantize(xd, _dev_scalar(gs_dev))
    p2, s2 = nv.quantize(xd, gs_host)
    assert np.array_equal(to_host(p1), to_host(p2)) and np.array_equal(to_host(s1), to_host(s2))
    wp, ws = O.quantize(x, gs_host)
    assert np.array_equal(to_host(p1), wp) and np.array_equal(to_host(s1), ws)


@pytest.mark.parametrize("M,N,K", [(2600, 1650, 128), (17, 3072, 256), (100, 130, 48), (4096, 4096, 128)])
def test_gemm_devgs_equals_gemm(M, N, K):
    rng = np.random.default_rng(M + N + K)
    x = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    ags, wgs = float(O.global_scale(x)), float(O.global_scale(w))
    ap, as_ = O.quantize(x, ags)
    wp, ws = O.quantize(w, wgs)
    say("gemm_devgs", nv.gemm_plan(M, N, K), M, N, K)
    args = (u8_to_dev(ap), u8_to_dev(as_))
    wargs = (u8_to_dev(wp), u8_to_dev(ws))
    o1 = nv.gemm(*args, _dev_scalar(ags), *wargs, _dev_scalar(wgs))
    o2 = nv.gemm(*args, ags, *wargs, wgs)
    assert np.array_equal(to_host(o1), to_host(o2))


@pytest.mark.parametrize("a_dev,w_dev,a_host,w_host", [
    (2.0**100, 2.0**-100, 2.0**90, 2.0**-90),      # clamped into [2^-90, 2^90]
    (float("nan"), 0.5, 1.0, 0.5), (-3.0, 0.0, 1.0, 1.0),
])
@pytest.mark.parametrize("M,N,K", [(2600, 1650, 128), (17, 3072, 256)])
def test_gemm_devgs_reads_scales_as_the_quantizer_does(M, N, K, a_dev, w_dev, a_host, w_host):
    """Device-resident GEMM scales outside [2^-90, 2^90] are clamped into it, NaN and
    values <= 0 read as 1.0 (as nvfp4_quantize_devgs reads its scale): the output equals
    nvfp4_gemm with the values so read, bit for bit."""
    rng = np.random.default_rng(M + K)
    codes = np.arange(0x30, 0x48, dtype=np.uint8)
    ap = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wp = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.choice(codes, (M, K // 16))
    ws = rng.choice(codes, (N, K // 16))
    say("gemm_devgs clamp", nv.gemm_plan(M, N, K), M, N, K, a_dev, w_dev)
    args = (u8_to_dev(ap), u8_to_dev(as_))
    wargs = (u8_to_dev(wp), u8_to_dev(ws))
    o1 = nv.gemm(*args, _dev_scalar(a_dev), *wargs, _dev_scalar(w_dev))
    o2 = nv.gemm(*args, a_host, *wargs, w_host)
    assert np.array_equal(to_host(o1), to_host(o2))


def test_linear_devgs_end_to_end():
    """Calibrate on the device, then the fused linear with both scales device-resident:
    identical to the host-scale linear, and within the GEMM bound of the oracle."""
    wl = make("odd_m256")
    d = wl.generate()
    xd, wd = bf16_to_dev(d["x"]), bf16_to_dev(d["w"])
    say("linear_devgs", wl.name)
    ags_d, wgs_d = nv.calibrate_device(xd), nv.calibrate_device(wd)
    wp, ws = nv.quantize(wd, wgs_d)
    out_d = nv.linear(xd, ags_d, wp, ws, wgs_d)
    ags, wgs = float(O.global_scale(d["x"])), float(O.global_scale(d["w"]))
    out_h = nv.linear(xd, ags, wp, ws, wgs)
    got = to_host(out_d)
    assert np.array_equal(got, to_host(out_h))
    ap, as_ = O.quantize(d["x"], ags)
    wpo, wso = O.quantize(d["w"], wgs)
    assert np.array_equal(to_host(wp), wpo) and np.array_equal(to_host(ws), wso)
    ref, absref = O.gemm_ref(ap, as_, ags, wpo, wso, wgs)
    assert O.check_gemm(got, ref, absref)[0]


def test_binding_rejects_mixed_scales():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    p, s = nv.quantize(x, 1.0)
    with pytest.raises(TypeError):
        nv.gemm(p, s, _dev_scalar(1.0), p, s, 1.0)
    with pytest.raises(TypeError):
        nv.quantize(x, torch.ones((2,), dtype=torch.float32, device="cuda"))
