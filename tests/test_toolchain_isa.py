"""Guard against a compiler hazard seen with this toolchain: per-element reads of the
fp4 -> f16 conversion's two-lane result can be folded to its low lane (probe: reading
h.x and h.y of one conversion compiled to {h.x, h.x}). The kernels only consume whole
vectors; this test checks the generated gfx950 code still converts every byte of
every packed word (all four byte selects, in equal numbers) in each kernel that
decodes, so a miscompiled decode is caught on a CPU before any GPU run."""
import os
import re
import subprocess
from collections import Counter

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    from nvfp4_block_scaled_02_amd import build as B

    out = str(tmp_path_factory.mktemp("isa") / "gemm.s")
    cmd = [B.hipcc(), *B.compile_flags(), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "gemm.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def _kernels(asm):
    """{kernel symbol: body} for every kernel in the assembly."""
    out = {}
    for m in re.finditer(r"^(_Z\w+):\s*;\s*@", asm, flags=re.M):
        start = m.end()
        end = asm.find("s_endpgm", start)
        out[m.group(1)] = asm[start:end]
    return out


def test_every_decoding_kernel_converts_all_four_bytes(gemm_asm):
    kernels = _kernels(gemm_asm)
    decoding = {k: v for k, v in kernels.items() if "v_cvt_scalef32_pk_f16_fp4" in v}
    assert any("gemm_kernel" in k for k in decoding), list(kernels)
    for name, body in decoding.items():
        sels = Counter()
        for line in body.splitlines():
            if "v_cvt_scalef32_pk_f16_fp4" in line:
                m = re.search(r"op_sel:\[(\d),(\d),\d\]", line)
                sels[(m.group(1), m.group(2)) if m else ("0", "0")] += 1
        assert len(sels) == 4 and len(set(sels.values())) == 1, (name, dict(sels))


@pytest.fixture(scope="module")
def w4a16_asm(tmp_path_factory):
    from nvfp4_block_scaled_02_amd import build as B

    out = str(tmp_path_factory.mktemp("isa") / "gemm_w4a16.s")
    cmd = [B.hipcc(), *B.compile_flags(), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "gemm_w4a16.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def test_w4a16_kernels_convert_all_four_bytes(w4a16_asm):
    """The W4A16 weight decode goes through the fp4 -> fp32 conversion: same check."""
    kernels = _kernels(w4a16_asm)
    decoding = {k: v for k, v in kernels.items() if "v_cvt_scalef32_pk_f32_fp4" in v}
    assert decoding and all("w4a16" in k for k in decoding), list(kernels)
    for name, body in decoding.items():
        sels = Counter()
        for line in body.splitlines():
            if "v_cvt_scalef32_pk_f32_fp4" in line:
                m = re.search(r"op_sel:\[(\d),(\d),\d\]", line)
                sels[(m.group(1), m.group(2)) if m else ("0", "0")] += 1
        assert len(sels) == 4 and len(set(sels.values())) == 1, (name, dict(sels))
