"""The C ABI from several host threads at once, each on its own HIP stream (the header's
thread-safety statement): every thread's results must equal a serial run bit for bit.
ctypes drops the GIL during the calls, so the launches really interleave."""
import threading

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_02_amd as nv
from gpu_helpers import say
from oracle import nvfp4_oracle as O
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256, 512), (300, 520, 384), (17, 3072, 3072), (1000, 768, 1024), (1, 4096, 1024)]


def test_concurrent_host_threads_on_own_streams():
    rng = np.random.default_rng(31)
    cases = []
    for M, N, K in SHAPES:
        x = to_bf16_bits((rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float32))
        w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        ags, wgs = O.global_scale(x), O.global_scale(w)
        wp, ws = O.quantize(w, wgs)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        cases.append((xd, float(ags), torch.from_numpy(wp).cuda(), torch.from_numpy(ws).cuda(), float(wgs)))
    say("concurrency: serial reference")
    ref = [nv.linear(*c) for c in cases]
    torch.cuda.synchronize()

    results = [None] * len(cases)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [nv.linear(*cases[i]) for _ in range(6)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported below
            errors.append((i, repr(e)))

    say("concurrency: threads", len(cases))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i, outs in enumerate(results):
        for o in outs:
            assert torch.equal(o.view(torch.int16), ref[i].view(torch.int16)), SHAPES[i]
