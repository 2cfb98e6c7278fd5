"""Ahead-of-time build of libnvfp4.so for gfx950 with hipcc (in-tree, no JIT).

``python -m nvfp4_block_scaled_02_amd.build`` (or ``build()``) compiles every HIP source
under ``csrc/`` into ``nvfp4_block_scaled_02_amd/libnvfp4.so``. Compilation happens on a
machine without a GPU: hipcc cross-compiles for gfx950.

Flags that matter for bit-exact rounding:
  -ffp-contract=off                     no fused multiply-adds beyond the explicit ones
  -fno-gpu-flush-denormals-to-zero      keep gradual underflow (f16 and fp32)
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division for '/'
and ``-target-feature -packed-fp32-ops`` keeps the compiler from emitting packed fp32
arithmetic.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "gemm_w4a16.hip", "mxfp8.hip", "fp8r.hip", "amax.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=off",
        "-fno-gpu-flush-denormals-to-zero",
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if err and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link libnvfp4.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
