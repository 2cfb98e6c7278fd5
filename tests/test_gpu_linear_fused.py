"""The fused linear for the shortest activations on the GPU: one kernel in which the
split-K GEMM first quantizes the bf16 activations into LDS (the quantize step of the pages'
fused quantize + FP4 GEMM pairing, "BFL (fp8r / nvfp4)", Kernels table, nvfp4 row).

For every shape the library routes to it (nvfp4_linear_plan), the workspace must be
bit-exact to the oracle's quantization, the output bit-identical to the two-kernel form
(nvfp4_gemm on those codes) and within the GEMM bound of the float64 reference; writes
must stay inside the workspace and the output. Covered: one row, ragged rows and
columns, K % 64 == 32 (a half-filled last chunk whose upper lanes read past their row),
long K, zero and -0 rows, a static input scale small enough that block scales saturate
(the clamped quotient), and device-resident global scales.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host, u8_to_dev
from oracle import nvfp4_oracle as O
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
    if M > 2:
        x[1] = 0.0
        x[2, ::3] = -0.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return to_bf16_bits(x), to_bf16_bits(w)


def _run_fused(x, ags, wp, ws, wgs, scale_dev=False):
    M, K = x.shape
    N = wp.shape[0]
    nbytes = nv.linear_workspace_bytes(M, K)
    work, ok_w = guarded((nbytes,), torch.uint8)
    out, ok_o = guarded((M, N), torch.bfloat16)
    a = torch.tensor([ags], dtype=torch.float32, device="cuda") if scale_dev else float(ags)
    b = torch.tensor([wgs], dtype=torch.float32, device="cuda") if scale_dev else float(wgs)
    nv.linear(bf16_to_dev(x), a, u8_to_dev(wp), u8_to_dev(ws), b, out=out, workspace=work)
    got = to_host(out)
    qp, qs = nv.workspace_views(work, M, K)
    assert ok_w() and ok_o(), "write outside the workspace or the output"
    return got, to_host(qp), to_host(qs)


def _check(x, w, ags, label, scale_dev=False):
    M, K = x.shape
    N = w.shape[0]
    assert nv.linear_plan(M, N, K) == "fused", label
    wgs = O.global_scale(w)
    wp, ws = O.quantize(w, wgs)
    say("linear fused", label, M, N, K, "device scales" if scale_dev else "")
    got, qp, qs = _run_fused(x, ags, wp, ws, wgs, scale_dev)
    ap, as_ = O.quantize(x, ags)
    assert np.array_equal(qp, ap), f"{label}: {np.count_nonzero(qp != ap)} packed bytes differ"
    assert np.array_equal(qs, as_), f"{label}: {np.count_nonzero(qs != as_)} scale bytes differ"
    two = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    nv.gemm(u8_to_dev(ap), u8_to_dev(as_), float(ags), u8_to_dev(wp), u8_to_dev(ws), float(wgs),
            out=two)
    assert np.array_equal(got, to_host(two)), f"{label}: differs from quantize + gemm"
    ref, absref = O.gemm_ref(ap, as_, ags, wp, ws, wgs)
    ok, worst, nbad = O.check_gemm(got, ref, absref)
    assert ok, f"{label}: {nbad} out of tolerance (worst {worst:.3g})"


@pytest.mark.parametrize("M,N,K", [
    (1, 3072, 3072), (5, 3072, 3072), (32, 200, 160), (5, 33, 96), (31, 1000, 224),
    (1, 64, 32), (3, 5000, 1056), (2, 96, 6144), (1, 3072, 12288), (16, 1024, 1024),
    (32, 12288, 512),
    # the 16-row kernel's fused form beyond 16384 elements (up to 24576)
    (6, 3072, 3072), (8, 3072, 3072), (24, 1024, 1024), (2, 96, 12288),
])
def test_fused_linear_matches_two_kernels(M, N, K):
    x, w = _inputs(M, N, K, M * 7 + N + K)
    _check(x, w, O.global_scale(x), f"{M}x{N}x{K}")


def test_fused_linear_saturating_static_scale():
    """An input scale 8x below calibration: the largest blocks' scales saturate at 448
    and their elements take the clamped quotient (codes saturate at 6)."""
    x, w = _inputs(20, 640, 512, 5)
    ags = np.float32(O.global_scale(x) / np.float32(8.0))
    ap, as_ = O.quantize(x, ags)
    assert np.count_nonzero(as_ == 0x7E) > 0
    _check(x, w, ags, "saturating")


def test_fused_linear_device_scales():
    x, w = _inputs(4, 3072, 3072, 6)
    _check(x, w, O.global_scale(x), "device scales", scale_dev=True)


def test_plan_boundary():
    """At most 32 rows and 16384 elements fuse (24576 on the 16-row kernel); just past
    either bound the linear runs as quantize + GEMM, with the same workspace contents."""
    assert nv.linear_plan(32, 3072, 512) == "fused"
    assert nv.linear_plan(32, 3072, 544) == "two_kernels"
    assert nv.linear_plan(33, 3072, 256) == "two_kernels"
    # the 16-row kernel (K % 256 == 0) fuses up to 24576 elements
    assert nv.linear_plan(32, 1024, 768) == "fused"
    assert nv.linear_plan(32, 1024, 1024) == "two_kernels"
    x, w = _inputs(33, 256, 256, 7)
    ags = O.global_scale(x)
    wgs = O.global_scale(w)
    wp, ws = O.quantize(w, wgs)
    say("linear two kernels", 33, 256, 256)
    got, qp, qs = _run_fused(x, ags, wp, ws, wgs)
    ap, as_ = O.quantize(x, ags)
    assert np.array_equal(qp, ap) and np.array_equal(qs, as_)
