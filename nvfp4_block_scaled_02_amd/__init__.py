"""libnvfp4: NVFP4 W4A4 linear layers with hand-written HIP kernels for MI355X (gfx950).

Python entry points (thin wrappers over the C ABI in include/nvfp4.h):

* :func:`quantize`  -- bf16 [M, K] -> packed E2M1 [M, K/2] + E4M3 scales [M, K/16]
* :func:`gemm`      -- block-scaled W4A4 GEMM, bf16 output
* :func:`linear`    -- fused quantize + GEMM through a workspace
* :func:`gemm_plan` -- which GEMM kernel a shape runs on (host only)
* :func:`gemm_w4a16_plan` -- the same for :func:`gemm_w4a16`
* :func:`linear_plan` -- whether :func:`linear` runs a shape as one fused kernel
* :func:`gemm_w4a16` -- NVFP4 weights x bf16 activations (not quantized), bf16 output
* :func:`mxfp8_quantize`, :func:`mxfp8_gemm` -- the MXFP8 (OCP microscaling) path
* :func:`fp8r_quantize`, :func:`fp8r_gemm` -- the rowwise FP8 path
* :func:`amax`, :func:`calibrate`, :func:`global_scale_from_amax` -- global scales
* :func:`calibrate_device` -- a global scale kept on the device (quantize, gemm and
  linear accept it in place of a float)
"""
from ._lib import NVFP4Error, load_library  # noqa: F401
from .ops import (  # noqa: F401
    amax,
    calibrate,
    calibrate_device,
    fp8r_gemm,
    fp8r_quantize,
    gemm,
    gemm_plan,
    gemm_w4a16,
    gemm_w4a16_plan,
    global_scale_from_amax,
    linear,
    linear_plan,
    linear_workspace_bytes,
    mxfp8_gemm,
    mxfp8_quantize,
    quantize,
    workspace_views,
)
