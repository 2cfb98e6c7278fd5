"""The quantizer's scalar codecs (csrc/codec.hpp), compiled for the host, against the
oracle. This checks the HIP path's rounding algorithms on a CPU; the GPU self-tests then
check that the device build and the conversion instructions give the same codes.
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import nvfp4_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "codec_host_check.cpp")
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_02_amd", "csrc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("codec") / "codec_host_check")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-ffp-contract=off", "-I", CSRC, SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    return r.stdout


def boundary_points(points, k=3):
    """float32 values within k ulps of each point (non-negative)."""
    p = np.asarray(points, dtype=np.float32)
    out = [p]
    up, dn = p, p
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up, dn]
    return np.concatenate(out)


def test_markstein_division_is_ieee_for_every_significand_pair(exe):
    out = _run(exe, "division")
    assert out.strip().endswith("mismatches 0"), out


def test_division_exact_at_extreme_exponents(exe):
    out = _run(exe, "extremes")
    assert out.strip().endswith("mismatches 0"), out


def test_e4m3_encoder_matches_oracle(exe, tmp_path):
    pos = O.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(1)
    s = np.concatenate([
        boundary_points(np.concatenate([pos, mids])),
        np.exp2(rng.uniform(-30, 20, 200_000)).astype(np.float32),
        np.float32([0.0, 447.99997, 448.0, 464.0, 465.0, 1e30, np.inf, 2.0**-149]),
    ]).astype(np.float32)
    s = s[s >= 0]
    inp, outp = tmp_path / "s.bin", tmp_path / "c.bin"
    s.tofile(inp)
    _run(exe, "e4m3", str(inp), str(outp))
    got = np.fromfile(outp, dtype=np.uint8)
    assert np.array_equal(got, O.e4m3_encode(s))


def test_e4m3_decoder_matches_oracle(exe, tmp_path):
    outp = tmp_path / "v.bin"
    _run(exe, "e4m3dec", str(outp))
    got = np.fromfile(outp, dtype=np.float32)
    assert np.array_equal(got.astype(np.float64), O.e4m3_decode(np.arange(127)))


def test_e2m1_software_encoder_matches_oracle(exe, tmp_path):
    g = np.float32([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6])
    rng = np.random.default_rng(2)
    y = np.concatenate([
        boundary_points(g, k=4),
        rng.uniform(0, 8, 100_000).astype(np.float32),
        np.exp2(rng.uniform(-149, 127, 20_000)).astype(np.float32),
        np.float32([np.inf, 3.4e38, 2.0**-149, 0.0]),
    ])
    y = np.concatenate([y, -y])  # includes -0.0 and negative infinities
    inp, outp = tmp_path / "y.bin", tmp_path / "c.bin"
    y.tofile(inp)
    _run(exe, "e2m1", str(inp), str(outp))
    got = np.fromfile(outp, dtype=np.uint8)
    want = (np.signbit(y).astype(np.uint8) << 3) | O.e2m1_encode_magnitude(np.abs(y))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("gs", [1.0, 2.0**-6, 1.0 / 3.0, 3.7e-4, 2.0**-90, 2.0**90, 0.0123])
def test_block_scale_matches_oracle(exe, tmp_path, gs):
    gs = np.float32(gs)
    den = np.float32(np.float32(6.0) * gs)
    pos = O.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    # amax values whose s_raw lands on or next to every E4M3 value and midpoint
    targets = np.concatenate([pos, mids]).astype(np.float64) * float(den)
    targets = targets[(targets > 0) & (targets < 3e38)].astype(np.float32)
    rng = np.random.default_rng(3)
    amax = np.concatenate([
        boundary_points(targets),
        (np.exp2(rng.uniform(-20, 20, 50_000)) * float(den)).astype(np.float32),
        np.float32([0.0, 2.0**-149, 3.3e38]),
    ])
    amax = amax[np.isfinite(amax) & (amax >= 0)]
    amax = (amax.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # bf16 values
    inp, outp = tmp_path / "a.bin", tmp_path / "o.bin"
    amax.tofile(inp)
    _run(exe, "scale", str(inp), "%08x" % int(gs.view(np.uint32)), str(outp))
    raw = np.fromfile(outp, dtype=np.uint8).reshape(-1, 5)
    code = raw[:, 0]
    d = raw[:, 1:].copy().view(np.float32)[:, 0]
    with np.errstate(over="ignore"):
        s_raw = (amax / den).astype(np.float32)
    want_code = O.e4m3_encode(s_raw)
    want_d = (O.e4m3_decode(want_code).astype(np.float32) * gs).astype(np.float32)
    assert np.array_equal(code, want_code)
    assert np.array_equal(d.view(np.uint32), want_d.view(np.uint32))
