"""Thin PyTorch-facing binding over libnvfp4's C ABI.

Argument marshalling only: each function checks tensor dtypes, shapes and devices, takes
the current HIP stream from PyTorch, passes raw pointers to the library and raises on a
non-zero status. Every step of the computation runs in the library's HIP kernels.
Function names follow the C entry points (include/nvfp4.h).
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import check, load_library


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dev_scale(v, name: str):
    """A device-resident global scale (a float32 tensor with one element) or None for a
    host float."""
    if not isinstance(v, torch.Tensor):
        return None
    if v.dtype != torch.float32 or v.numel() != 1:
        raise TypeError(f"{name} as a tensor must be float32 with one element")
    if not v.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    return v


def quantize(x: torch.Tensor, global_scale, packed: torch.Tensor | None = None,
             scales: torch.Tensor | None = None, stream=None):
    """NVFP4-quantize bf16 ``x`` [M, K] -> (packed uint8 [M, K/2], scales uint8 [M, K/16]).

    ``global_scale`` is a float, or a device float32 tensor of one element (read by the
    kernel, no host round trip; see :func:`calibrate_device`)."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    if packed is None:
        packed = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _need(packed, "packed", torch.uint8, 2)
    _need(scales, "scales", torch.uint8, 2)
    if tuple(packed.shape) != (M, K // 2) or tuple(scales.shape) != (M, K // 16):
        raise ValueError("output shapes do not match x")
    lib = load_library()
    gsd = _dev_scale(global_scale, "global_scale")
    if gsd is not None:
        check(lib.nvfp4_quantize_devgs(_ptr(x), M, K, _ptr(gsd), _ptr(packed), _ptr(scales),
                                       _stream(stream)), "nvfp4_quantize_devgs")
    else:
        check(lib.nvfp4_quantize(_ptr(x), M, K, float(global_scale), _ptr(packed), _ptr(scales),
                                 _stream(stream)), "nvfp4_quantize")
    return packed, scales


def gemm(a_packed: torch.Tensor, a_scales: torch.Tensor, a_global_scale,
         w_packed: torch.Tensor, w_scales: torch.Tensor, w_global_scale,
         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Block-scaled W4A4 GEMM: bf16 [M, N] = a_gs * w_gs * A_hat @ W_hat^T. The global
    scales are both floats or both device float32 tensors of one element."""
    for t, n in ((a_packed, "a_packed"), (a_scales, "a_scales"), (w_packed, "w_packed"),
                 (w_scales, "w_scales")):
        _need(t, n, torch.uint8, 2)
    M, Kh = a_packed.shape
    N = w_packed.shape[0]
    K = 2 * Kh
    if tuple(w_packed.shape) != (N, Kh) or tuple(a_scales.shape) != (M, K // 16) or \
            tuple(w_scales.shape) != (N, K // 16):
        raise ValueError("operand shapes are inconsistent")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_packed.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape must be [M, N]")
    lib = load_library()
    ad, wd = _dev_scale(a_global_scale, "a_global_scale"), _dev_scale(w_global_scale, "w_global_scale")
    if (ad is None) != (wd is None):
        raise TypeError("global scales must be both floats or both device tensors")
    if ad is not None:
        check(lib.nvfp4_gemm_devgs(_ptr(a_packed), _ptr(a_scales), _ptr(ad), _ptr(w_packed),
                                   _ptr(w_scales), _ptr(wd), M, N, K, _ptr(out), _stream(stream)),
              "nvfp4_gemm_devgs")
    else:
        check(lib.nvfp4_gemm(_ptr(a_packed), _ptr(a_scales), float(a_global_scale), _ptr(w_packed),
                             _ptr(w_scales), float(w_global_scale), M, N, K, _ptr(out),
                             _stream(stream)), "nvfp4_gemm")
    return out


def gemm_w4a16(x: torch.Tensor, w_packed: torch.Tensor, w_scales: torch.Tensor,
               w_global_scale: float, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """W4A16 GEMM: bf16 [M, N] = w_gs * x @ W_hat^T with x bf16 (not quantized)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_packed, "w_packed", torch.uint8, 2)
    _need(w_scales, "w_scales", torch.uint8, 2)
    M, K = x.shape
    N = w_packed.shape[0]
    if tuple(w_packed.shape) != (N, K // 2) or tuple(w_scales.shape) != (N, K // 16):
        raise ValueError("weight shapes do not match x")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape must be [M, N]")
    lib = load_library()
    check(lib.nvfp4_gemm_w4a16(_ptr(x), _ptr(w_packed), _ptr(w_scales), float(w_global_scale),
                               M, N, K, _ptr(out), _stream(stream)), "nvfp4_gemm_w4a16")
    return out


_MX_ELEMENTS = {"e4m3": 0, "e5m2": 1}


def _mx_element(elem: str) -> int:
    if elem not in _MX_ELEMENTS:
        raise ValueError(f"MXFP8 element type must be one of {sorted(_MX_ELEMENTS)}, not {elem!r}")
    return _MX_ELEMENTS[elem]


def mxfp8_quantize(x: torch.Tensor, codes: torch.Tensor | None = None,
                   scales: torch.Tensor | None = None, stream=None, elem: str = "e4m3"):
    """MXFP8 quantization: bf16 [M, K] -> E4M3 or E5M2 codes uint8 [M, K] + E8M0 scales
    [M, K/32]."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _need(codes, "codes", torch.uint8, 2)
    _need(scales, "scales", torch.uint8, 2)
    if tuple(codes.shape) != (M, K) or tuple(scales.shape) != (M, K // 32):
        raise ValueError("codes must be [M, K] and scales [M, K/32]")
    lib = load_library()
    check(lib.nvfp4_mxfp8_quantize_elem(_ptr(x), M, K, _mx_element(elem), _ptr(codes), _ptr(scales),
                                        _stream(stream)), "nvfp4_mxfp8_quantize_elem")
    return codes, scales


def mxfp8_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
               w_scales: torch.Tensor, out: torch.Tensor | None = None, stream=None,
               a_elem: str = "e4m3", w_elem: str = "e4m3") -> torch.Tensor:
    """MXFP8 GEMM: bf16 [M, N] = A_hat @ W_hat^T on the block-scaled fp8 MFMA (each operand
    E4M3 or E5M2)."""
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (w_codes, "w_codes"),
                 (w_scales, "w_scales")):
        _need(t, n, torch.uint8, 2)
    M, K = a_codes.shape
    N = w_codes.shape[0]
    if tuple(w_codes.shape) != (N, K) or tuple(a_scales.shape) != (M, K // 32) or \
            tuple(w_scales.shape) != (N, K // 32):
        raise ValueError("operand shapes are inconsistent")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape must be [M, N]")
    lib = load_library()
    check(lib.nvfp4_mxfp8_gemm_elem(_ptr(a_codes), _ptr(a_scales), _mx_element(a_elem), _ptr(w_codes),
                                    _ptr(w_scales), _mx_element(w_elem), M, N, K, _ptr(out),
                                    _stream(stream)), "nvfp4_mxfp8_gemm_elem")
    return out


def fp8r_quantize(x: torch.Tensor, codes: torch.Tensor | None = None,
                  scales: torch.Tensor | None = None, stream=None):
    """Rowwise FP8 quantization: bf16 [M, K] -> E4M3 codes uint8 [M, K] + fp32 scales [M]."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8, 2)
    _need(scales, "scales", torch.float32, 1)
    if tuple(codes.shape) != (M, K) or tuple(scales.shape) != (M,):
        raise ValueError("codes must be [M, K] and scales [M]")
    lib = load_library()
    check(lib.nvfp4_fp8r_quantize(_ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(stream)),
          "nvfp4_fp8r_quantize")
    return codes, scales


def fp8r_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Rowwise FP8 GEMM: bf16 [M, N] = diag(a_scales) Qa Qw^T diag(w_scales)."""
    _need(a_codes, "a_codes", torch.uint8, 2)
    _need(w_codes, "w_codes", torch.uint8, 2)
    _need(a_scales, "a_scales", torch.float32, 1)
    _need(w_scales, "w_scales", torch.float32, 1)
    M, K = a_codes.shape
    N = w_codes.shape[0]
    if tuple(w_codes.shape) != (N, K) or tuple(a_scales.shape) != (M,) or \
            tuple(w_scales.shape) != (N,):
        raise ValueError("operand shapes are inconsistent")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape must be [M, N]")
    lib = load_library()
    check(lib.nvfp4_fp8r_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales),
                              M, N, K, _ptr(out), _stream(stream)), "nvfp4_fp8r_gemm")
    return out


GEMM_KERNELS = {0: "tile256", 1: "fit", 2: "splitk", 3: "generic", 4: "tile128", 5: "tile128x128", 6: "tile128x64",
                7: "wsplit64", 8: "wsplit128", 9: "gemv16"}


def gemm_plan(M: int, N: int, K: int, num_cus: int = 0) -> str:
    """Name of the kernel :func:`gemm` launches for an M x N x K product with aligned
    operands on a device with ``num_cus`` compute units (0: 256, an MI355X). Host only."""
    kind = ctypes.c_int(-1)
    check(load_library().nvfp4_gemm_plan(M, N, K, num_cus, ctypes.byref(kind)), "nvfp4_gemm_plan")
    return GEMM_KERNELS[kind.value]


W4A16_KERNELS = {0: "splitk", 1: "fit", 2: "tile256", 3: "wide", 4: "wide128x256", 5: "wide96x256",
                 6: "wide128x128", 7: "wide64x128", 8: "gemv16"}


def gemm_w4a16_plan(M: int, N: int, K: int, num_cus: int = 0) -> str:
    """Name of the kernel :func:`gemm_w4a16` launches for an M x N x K product on a device
    with ``num_cus`` compute units (0: 256, an MI355X). Host only."""
    kind = ctypes.c_int(-1)
    check(load_library().nvfp4_gemm_w4a16_plan(M, N, K, num_cus, ctypes.byref(kind)), "nvfp4_gemm_w4a16_plan")
    return W4A16_KERNELS[kind.value]


def linear_plan(M: int, N: int, K: int, num_cus: int = 0) -> str:
    """"fused" when :func:`linear` runs the shape as one kernel (quantize inside the
    short-activation GEMM), else "two_kernels". Host only."""
    fused = ctypes.c_int(-1)
    check(load_library().nvfp4_linear_plan(M, N, K, num_cus, ctypes.byref(fused)), "nvfp4_linear_plan")
    return "fused" if fused.value == 1 else "two_kernels"


def linear_workspace_bytes(M: int, K: int) -> int:
    return int(load_library().nvfp4_linear_workspace_bytes(M, K))


def linear(x: torch.Tensor, a_global_scale, w_packed: torch.Tensor,
           w_scales: torch.Tensor, w_global_scale, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fused NVFP4 linear: quantize x under a_global_scale, then the W4A4 GEMM. The global
    scales are both floats or both device float32 tensors of one element."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_packed, "w_packed", torch.uint8, 2)
    _need(w_scales, "w_scales", torch.uint8, 2)
    M, K = x.shape
    N = w_packed.shape[0]
    if tuple(w_packed.shape) != (N, K // 2) or tuple(w_scales.shape) != (N, K // 16):
        raise ValueError("weight shapes do not match x")
    need = linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape must be [M, N]")
    lib = load_library()
    ad, wd = _dev_scale(a_global_scale, "a_global_scale"), _dev_scale(w_global_scale, "w_global_scale")
    if (ad is None) != (wd is None):
        raise TypeError("global scales must be both floats or both device tensors")
    if ad is not None:
        check(lib.nvfp4_linear_devgs(_ptr(x), _ptr(ad), _ptr(w_packed), _ptr(w_scales), _ptr(wd),
                                     M, N, K, _ptr(out), _ptr(workspace), workspace.numel(),
                                     _stream(stream)), "nvfp4_linear_devgs")
    else:
        check(lib.nvfp4_linear(_ptr(x), float(a_global_scale), _ptr(w_packed), _ptr(w_scales),
                               float(w_global_scale), M, N, K, _ptr(out), _ptr(workspace),
                               workspace.numel(), _stream(stream)), "nvfp4_linear")
    return out


def workspace_views(workspace: torch.Tensor, M: int, K: int):
    """(packed [M, K/2], scales [M, K/16]) views of a linear() workspace (layout of
    nvfp4_linear: packed at 0, scales at round_up(M*K/2, 256))."""
    off = (M * K // 2 + 255) // 256 * 256
    packed = workspace[: M * K // 2].view(M, K // 2)
    scales = workspace[off: off + M * K // 16].view(M, K // 16)
    return packed, scales


def amax(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Device fp32 [1] tensor holding max |x| over a bf16 tensor (any shape, contiguous)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 HIP tensor")
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=x.device)
    lib = load_library()
    check(lib.nvfp4_amax(_ptr(x), x.numel(), _ptr(out), _stream(stream)), "nvfp4_amax")
    return out


def global_scale_from_amax(a: float) -> float:
    """RN32(amax / 2688) computed by the library (1.0 for amax == 0)."""
    return float(load_library().nvfp4_global_scale_from_amax(float(a)))


def calibrate_device(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Global scale of a bf16 tensor computed and kept on the device: a float32 tensor of
    one element holding RN32(amax / 2688) clamped into [2^-90, 2^90] (1 for an all-zero
    tensor). Asynchronous; pass it straight to :func:`quantize`, :func:`gemm` or
    :func:`linear`."""
    _need(x, "x", torch.bfloat16, x.dim())
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=x.device)
    _dev_scale(out, "out")
    check(load_library().nvfp4_calibrate_device(_ptr(x), x.numel(), _ptr(out), _stream(stream)),
          "nvfp4_calibrate_device")
    return out


def calibrate(x: torch.Tensor, stream=None) -> float:
    """Global scale of a bf16 tensor: device amax, read back (synchronises), then
    RN32(amax / 2688). Used once per tensor, offline (weights) or at calibration time
    (static activation scale)."""
    a = amax(x, stream=stream)
    return global_scale_from_amax(float(a.item()))
