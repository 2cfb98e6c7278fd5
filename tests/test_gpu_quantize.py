"""nvfp4_quantize on the GPU: bit-exact against the CPU oracle (packed bytes and scale
bytes) on every FLUX-shaped workload at full size, on weights and activations, and on
adversarial and ragged inputs. Calibration (amax, global scale) is bit-exact too."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host
from oracle import nvfp4_oracle as O
from workloads import make, names, to_bf16_bits

pytestmark = pytest.mark.gpu


def _check_quantize(x_bits, gs, label):
    say("quantize", label, x_bits.shape, float(gs))
    M, K = x_bits.shape
    xd = bf16_to_dev(x_bits)
    p, pc = guarded((M, K // 2), torch.uint8)
    s, sc = guarded((M, K // 16), torch.uint8)
    nv.quantize(xd, float(gs), packed=p, scales=s)
    gp, gsc = to_host(p), to_host(s)
    assert pc() and sc(), "write outside the output buffers"
    wp, ws = O.quantize(x_bits, gs)
    bad = np.argwhere(gp != wp)
    assert np.array_equal(gsc, ws), (label, np.argwhere(gsc != ws)[:5])
    detail = [(int(r), int(c), hex(int(gp[r, c])), hex(int(wp[r, c])),
               [hex(int(v)) for v in x_bits[r, 2 * c: 2 * c + 2]]) for r, c in bad[:5]]
    assert bad.size == 0, (label, len(bad), detail)
    return p, s


@pytest.mark.parametrize("name", names())
def test_workload_activations_and_weights_bit_exact(name):
    wl = make(name)
    d = wl.generate()
    # calibration through the library (device amax + host RN32 division)
    calib = d.get("calib", d["x"])
    ags = nv.calibrate(bf16_to_dev(calib))
    assert np.float32(ags).view(np.uint32) == O.global_scale(calib).view(np.uint32)
    wgs = nv.calibrate(bf16_to_dev(d["w"]))
    assert np.float32(wgs).view(np.uint32) == O.global_scale(d["w"]).view(np.uint32)
    _check_quantize(d["x"], np.float32(ags), name + "/x")
    _check_quantize(d["w"], np.float32(wgs), name + "/w")


def test_amax_exact_on_odd_lengths():
    rng = np.random.default_rng(5)
    for n in [1, 7, 8, 9, 1000, 4097, 123457, 3000001]:
        v = to_bf16_bits((rng.standard_normal(n) * np.exp(rng.uniform(-5, 5))).astype(np.float32))
        say("amax", n)
        got = to_host(nv.amax(bf16_to_dev(v)))[0]
        assert got == np.abs(O.bf16_bits_to_f32(v)).max()
    z = np.zeros(64, np.uint16)
    z[3] = 0x8000
    assert to_host(nv.amax(bf16_to_dev(z)))[0] == 0.0


def _adversarial(rng, M, K):
    cases = {}
    g = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], np.float32)
    v = rng.choice(g, size=(M, K)) * rng.choice([-1, 1], size=(M, K)).astype(np.float32)
    v *= (2.0 ** rng.integers(-8, 8, size=(M, 1))).astype(np.float32)
    cases["grid_and_ties"] = to_bf16_bits(v)
    z = rng.standard_normal((M, K)).astype(np.float32)
    z[:, :16] = 0.0
    z[:, 16:32] = -0.0
    z[1::3, 32:48] *= np.float32(2.0**-30)
    cases["zero_and_tiny_blocks"] = to_bf16_bits(z)
    h = rng.standard_t(1.0, size=(M, K)).astype(np.float32)
    cases["cauchy"] = to_bf16_bits(np.clip(h, -3e38, 3e38))
    cases["row_scales"] = to_bf16_bits(
        (rng.standard_normal((M, K)) * np.exp2(rng.uniform(-60, 60, (M, 1)))).astype(np.float32))
    return cases


@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (5, 80), (64, 256), (257, 1040)])
def test_adversarial_and_ragged(M, K):
    rng = np.random.default_rng(M * 7 + K)
    for label, x in _adversarial(rng, M, K).items():
        gs = O.global_scale(x)
        _check_quantize(x, gs, f"{label} {M}x{K} self")
        # static scales that are too small (E4M3 and E2M1 saturation) and too large
        # (E4M3 subnormal scales, scale underflow to 0)
        for f in (2.0**-12, 0.37, 2.0**9, 2.0**40):
            g2 = np.float32(np.clip(np.float32(gs) * np.float32(f), 2.0**-90, 2.0**90))
            _check_quantize(x, g2, f"{label} {M}x{K} x{f}")


def test_non_default_stream_and_determinism():
    rng = np.random.default_rng(9)
    x = to_bf16_bits(rng.standard_normal((512, 3072)).astype(np.float32))
    gs = O.global_scale(x)
    xd = bf16_to_dev(x)
    s = torch.cuda.Stream()
    say("quantize on a side stream")
    with torch.cuda.stream(s):
        p1, s1 = nv.quantize(xd, float(gs))
    s.synchronize()
    p2, s2 = nv.quantize(xd, float(gs))
    assert np.array_equal(to_host(p1), to_host(p2)) and np.array_equal(to_host(s1), to_host(s2))
    wp, ws = O.quantize(x, gs)
    assert np.array_equal(to_host(p1), wp) and np.array_equal(to_host(s1), ws)


def test_binding_rejects_bad_arguments():
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        nv.quantize(x, 1.0)
    x = torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        nv.quantize(x, 0.0)
    with pytest.raises(TypeError):
        nv.quantize(x.float(), 1.0)
