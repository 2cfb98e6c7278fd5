"""The hot path under HIP graph capture: device calibration of the input scale, then the
linear (quantize + GEMM, or the fused kernel for the shortest activations), captured
once and replayed with new inputs copied in eagerly between replays. Every replay must
equal the eager calls bit for bit. No step records a memset (the calibration clears its
counter with a kernel), so replays after the first see the same work as the first."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import say
from oracle import nvfp4_oracle as O
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(4608, 3072, 3072), (300, 512, 1024), (1, 3072, 3072), (17, 640, 256),
                                   (17, 3072, 3072), (17, 640, 160), (64, 3072, 1056)])
def test_linear_graph_replays_match_eager(M, N, K):
    rng = np.random.default_rng(M + N + K)
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wgs = O.global_scale(w)
    wp, ws = O.quantize(w, wgs)
    wp, ws = torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda()
    wgs_d = torch.tensor([float(wgs)], dtype=torch.float32, device="cuda")
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(nv.linear_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(M * 3 + K)

    def fill(i):
        x.copy_((torch.randn((M, K), device="cuda", generator=gen) * (1.0 + i)).to(torch.bfloat16))

    fill(0)
    say("graph capture", M, N, K, nv.gemm_plan(M, N, K), nv.linear_plan(M, N, K))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        a = nv.calibrate_device(x)
        nv.linear(x, a, wp, ws, wgs_d, workspace=work)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ags_g = nv.calibrate_device(x)
        out_g = nv.linear(x, ags_g, wp, ws, wgs_d, workspace=work)
    for i in range(4):
        fill(i + 1)
        g.replay()
        torch.cuda.synchronize()
        got = out_g.clone()
        ags_e = nv.calibrate_device(x)
        want = nv.linear(x, ags_e, wp, ws, wgs_d)
        torch.cuda.synchronize()
        assert torch.equal(ags_g, ags_e), i
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {i}"
