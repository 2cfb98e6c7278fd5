"""Synthetic FLUX-shaped linear-layer workloads (seeded, bf16 storage).

The pages print no layer shapes; these are the shapes of a FLUX-style diffusion
transformer block with hidden size 3072, MLP width 12288, fused QKV width 9216 and
M = 4096 image + 512 text tokens per image. Trained weights, prompts and images are
not available, so seeded random tensors of those shapes stand in for them.

Recipe (one fresh ``numpy.random.default_rng(seed)`` per workload; draws in the order
activations, weights, extras; float32 draws rounded to bf16 by PyTorch's CPU cast,
round-to-nearest-even):

* weights: N(0, 0.02^2) (standard deviation 0.02), layout [N, K].
* ``normal``: activations N(0, 1).
* ``outliers``: N(0, 1), then round(0.001 * M * K) distinct positions scaled by 20.
* ``student_t``: Student-t with 4 degrees of freedom divided by sqrt(2) (unit variance).
* ``lognormal_rows``: row magnitude exp(z), z ~ N(0, 1) per row, times N(0, 1).
* ``static`` scale: a second activation tensor of the same shape and distribution is
  drawn from ``default_rng(seed + 1)`` for offline calibration of the activation
  global scale; the live tensor is then quantised under that fixed scale.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE, PyTorch CPU cast); return raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str = "normal"  # normal | outliers | student_t | lognormal_rows
    static_scale: bool = False
    seed: int = 0
    description: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def _acts(self, rng: np.random.Generator, M: int) -> np.ndarray:
        K = self.K
        if self.dist in ("normal", "outliers"):
            return rng.standard_normal((M, K), dtype=np.float32)
        if self.dist == "student_t":
            return (rng.standard_t(4.0, size=(M, K)) / np.sqrt(2.0)).astype(np.float32)
        if self.dist == "lognormal_rows":
            z = rng.standard_normal(M, dtype=np.float32)
            base = rng.standard_normal((M, K), dtype=np.float32)
            return base * np.exp(z)[:, None]
        raise ValueError(self.dist)

    def generate(self, with_weights: bool = True):
        """Return dict with ``x`` (uint16 [M,K]), ``w`` (uint16 [N,K]) and optionally
        ``calib`` (uint16 [M,K], for a static activation scale)."""
        rng = np.random.default_rng(self.seed)
        x = self._acts(rng, self.M)
        out = {}
        if with_weights:
            w = rng.standard_normal((self.N, self.K), dtype=np.float32) * np.float32(0.02)
            out["w"] = to_bf16_bits(w)
            del w
        if self.dist == "outliers":
            n_out = int(round(0.001 * self.M * self.K))
            pos = rng.choice(self.M * self.K, size=n_out, replace=False)
            flat = x.reshape(-1)
            flat[pos] *= np.float32(20.0)
        out["x"] = to_bf16_bits(x)
        del x
        if self.static_scale:
            crng = np.random.default_rng(self.seed + 1)
            out["calib"] = to_bf16_bits(self._acts(crng, self.M))
        return out


def _wl(*a, **k) -> Workload:
    return Workload(*a, **k)


# Shapes of the FLUX block linears (M = 4096 image + 512 text tokens).
WORKLOADS = {
    w.name: w
    for w in [
        _wl("tiny", 64, 128, 256, description="tiny NVFP4 linear, x~N(0,1)"),
        _wl("attn_out", 4608, 3072, 3072, dist="outliers",
            description="attention out-projection, 0.1% outliers x20"),
        _wl("mlp_up_static", 4608, 12288, 3072, static_scale=True,
            description="MLP up-projection, static (pre-calibrated) activation scale"),
        _wl("qkv", 4608, 9216, 3072, dist="student_t",
            description="fused QKV projection, Student-t(4) activations"),
        _wl("mlp_down", 4608, 3072, 12288, dist="student_t",
            description="MLP down-projection (K=12288), Student-t(4) activations"),
        _wl("batch4_up", 18432, 12288, 3072, dist="lognormal_rows",
            description="4-image batch MLP up-projection, LogNormal row magnitudes"),
        _wl("odd_m1", 1, 3072, 3072, dist="lognormal_rows", description="M=1"),
        _wl("odd_m17", 17, 3072, 3072, dist="lognormal_rows", description="M=17"),
        _wl("odd_m256", 256, 3072, 3072, dist="lognormal_rows", description="M=256"),
        _wl("odd_m1000", 1000, 3072, 3072, dist="lognormal_rows", description="M=1000"),
    ]
}


def names():
    return list(WORKLOADS)


def make(name: str) -> Workload:
    return WORKLOADS[name]
