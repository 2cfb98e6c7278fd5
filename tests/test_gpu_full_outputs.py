"""Every output element of every workload at full size, against the CPU oracle.

Each workload runs once through ``nvfp4_linear`` (the quantize kernel into the
workspace, then the GEMM kernel the planner picks: the bench's launch configuration) on
its seeded tensors. The workspace must equal the oracle's quantization bit for bit, the
output must equal ``nvfp4_gemm`` on that workspace bit for bit (and a second launch), and
every output element must lie within 2^-10 * sum_k |a_k w_k| + 1 bf16 ulp of the exact
float64 product. The comparison runs in row chunks (one test case each, so progress shows
as the cases finish), with the decoded weights computed once per workload.

The flagship shape (4608 x 3072 x 3072) also runs in full through the next-row paths:
W4A16, MXFP8 and the rowwise FP8 GEMM.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import bf16_to_dev, guarded, say, to_host, u8_to_dev
from oracle import fp8r_oracle as FR
from oracle import mxfp8_oracle as MX
from oracle import nvfp4_oracle as O
from workloads import make

pytestmark = pytest.mark.gpu

CHUNK = 1152  # rows per comparison case (4608 = 4 chunks, 18432 = 16)
WORKLOADS = ["tiny", "odd_m1", "odd_m17", "odd_m256", "odd_m1000",
             "attn_out", "mlp_up_static", "qkv", "mlp_down", "batch4_up"]


def _cases():
    out = []
    for name in WORKLOADS:
        M = make(name).M
        out += [(name, c) for c in range((M + CHUNK - 1) // CHUNK)]
    return out


_RUN = {}


def _run(name):
    """Device results and oracle operands of one workload (kept until the next one)."""
    if name in _RUN:
        return _RUN[name]
    _RUN.clear()
    wl = make(name)
    d = wl.generate()
    ags = O.global_scale(d.get("calib", d["x"]))
    wgs = O.global_scale(d["w"])
    wp, ws = O.quantize(d["w"], wgs)
    ap, as_ = O.quantize(d["x"], ags)
    M, N, K = wl.M, wl.N, wl.K
    say("full-output linear", name, M, N, K, "gemm kernel", nv.gemm_plan(M, N, K),
        "linear", nv.linear_plan(M, N, K))
    # output and workspace inside canary bytes: nothing is written outside them
    work, work_guard = guarded((nv.linear_workspace_bytes(M, K),), torch.uint8)
    out, out_guard = guarded((M, N), torch.bfloat16)
    wpd, wsd = u8_to_dev(wp), u8_to_dev(ws)
    nv.linear(bf16_to_dev(d["x"]), float(ags), wpd, wsd, float(wgs), out=out, workspace=work)
    got = to_host(out)
    guards_ok = work_guard() and out_guard()
    qp, qs = nv.workspace_views(work, M, K)
    ws_ok = np.array_equal(to_host(qp), ap) and np.array_equal(to_host(qs), as_)
    # the GEMM alone on the workspace, twice: bit-identical to the linear's output
    same = True
    for _ in range(2):
        g = nv.gemm(qp, qs, float(ags), wpd, wsd, float(wgs))
        same = same and np.array_equal(to_host(g), got)
        del g
    del out, work, qp, qs, wpd, wsd
    torch.cuda.empty_cache()
    r = dict(M=M, got=got, ap=ap, as_=as_, ags=ags, wgs=wgs, wp=wp, ws=ws, ws_ok=ws_ok,
             same=same, guards_ok=guards_ok, W=O.decode_blocks(wp, ws))
    _RUN[name] = r
    return r


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,chunk", _cases())
def test_linear_every_output_element(name, chunk):
    r = _run(name)
    if chunk == 0:
        assert r["ws_ok"], f"{name}: workspace differs from the oracle's quantization"
        assert r["same"], f"{name}: nvfp4_gemm on the workspace differs from nvfp4_linear"
        assert r["guards_ok"], f"{name}: bytes written outside the output or the workspace"
    r0, r1 = chunk * CHUNK, min(r["M"], (chunk + 1) * CHUNK)
    ref, absref = O.gemm_ref(r["ap"][r0:r1], r["as_"][r0:r1], r["ags"], r["wp"], r["ws"], r["wgs"],
                             w_decoded=r["W"])
    ok, worst, nbad = O.check_gemm(r["got"][r0:r1], ref, absref)
    assert ok, f"{name} rows {r0}:{r1}: {nbad} out of tolerance (worst err/tol {worst:.3g})"


def _flagship():
    wl = make("attn_out")
    return wl, wl.generate()


@pytest.mark.timeout(600)
def test_w4a16_flagship_every_output_element():
    wl, d = _flagship()
    wgs = O.global_scale(d["w"])
    wp, ws = O.quantize(d["w"], wgs)
    say("full-output w4a16 attn_out")
    got = to_host(nv.gemm_w4a16(bf16_to_dev(d["x"]), u8_to_dev(wp), u8_to_dev(ws), float(wgs)))
    for r0 in range(0, wl.M, CHUNK):
        r1 = min(wl.M, r0 + CHUNK)
        ref, absref = O.w4a16_ref(d["x"][r0:r1], wp, ws, wgs)
        ok, worst, nbad = O.check_gemm(got[r0:r1], ref, absref)
        assert ok, f"rows {r0}:{r1}: {nbad} out of tolerance (worst {worst:.3g})"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("a_elem,w_elem", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e5m2", "e4m3")])
def test_mxfp8_flagship_every_output_element(a_elem, w_elem):
    wl, d = _flagship()
    ac, as_ = MX.quantize(d["x"], elem=a_elem)
    wc, ws = MX.quantize(d["w"], elem=w_elem)
    say("full-output mxfp8 attn_out", a_elem, w_elem)
    acd, asd = nv.mxfp8_quantize(bf16_to_dev(d["x"]), elem=a_elem)
    assert np.array_equal(to_host(acd), ac) and np.array_equal(to_host(asd), as_)
    got = to_host(nv.mxfp8_gemm(acd, asd, u8_to_dev(wc), u8_to_dev(ws), a_elem=a_elem, w_elem=w_elem))
    for r0 in range(0, wl.M, CHUNK):
        r1 = min(wl.M, r0 + CHUNK)
        ref, absref = MX.gemm_ref(ac[r0:r1], as_[r0:r1], wc, ws, a_elem=a_elem, w_elem=w_elem)
        ok, worst, nbad = O.check_gemm(got[r0:r1], ref, absref)
        assert ok, f"rows {r0}:{r1}: {nbad} out of tolerance (worst {worst:.3g})"


@pytest.mark.timeout(600)
def test_fp8r_flagship_every_output_element():
    wl, d = _flagship()
    ac, as_ = FR.quantize(d["x"])
    wc, ws = FR.quantize(d["w"])
    say("full-output fp8r attn_out")
    acd, asd = nv.fp8r_quantize(bf16_to_dev(d["x"]))
    assert np.array_equal(to_host(acd), ac) and np.array_equal(to_host(asd), as_)
    wsd = torch.from_numpy(np.ascontiguousarray(ws, dtype=np.float32)).to("cuda")
    got = to_host(nv.fp8r_gemm(acd, asd, u8_to_dev(wc), wsd))
    for r0 in range(0, wl.M, CHUNK):
        r1 = min(wl.M, r0 + CHUNK)
        ref, absref = FR.gemm_ref(ac[r0:r1], as_[r0:r1], wc, ws)
        ok, worst, nbad = O.check_gemm(got[r0:r1], ref, absref)
        assert ok, f"rows {r0}:{r1}: {nbad} out of tolerance (worst {worst:.3g})"
