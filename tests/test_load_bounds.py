"""Range-checked operand loads of the GEMM kernels, modelled on the CPU.

The tiled and split-K kernels read the ragged last tile's missing rows through buffer
loads that the hardware range-checks, so that those rows read as zero. The check covers
only the per-lane offset, not the scalar one, so each load must carry its row in the
per-lane offset. ``tests/native/load_bounds_check.cpp`` evaluates, on the host, the
same offset helpers the kernels call (``csrc/gemm_common.hpp``) for every tile, piece,
lane, position along K and dword of ragged shapes, and checks that no in-range dword
lies past the end of an exactly sized operand, that every byte of a real row is read
in range from its own address, and that rows past the end read as zero.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "load_bounds_check.cpp")
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_02_amd", "csrc")


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("loads") / "load_bounds_check")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-I", CSRC, "-I", os.path.join(ROOT, "include"), SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    return r


@pytest.mark.parametrize("family", ["nvfp4-code-pieces", "nvfp4-scale-pieces", "splitk", "gemv16", "w4a16-gemv16", "mxfp8",
                                    "w4a16-tiled", "w4a16-splitk"])
def test_no_load_leaves_its_operand(report, family):
    lines = {l.split(" loads ")[0]: l for l in report.stdout.splitlines() if " loads " in l}
    assert family in lines, report.stdout + report.stderr
    loads, bad = lines[family].split(" loads ")[1].split(" violations ")
    assert int(loads) > 0
    assert int(bad) == 0, lines[family] + "\n" + report.stderr


def test_model_exit_status(report):
    assert report.returncode == 0, report.stdout + report.stderr
