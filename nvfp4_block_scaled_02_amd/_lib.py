"""ctypes loader for libnvfp4.so (the C ABI in include/nvfp4.h and include/nvfp4_selftest.h).

The library is built ahead of time, in-tree, by ``nvfp4_block_scaled_02_amd.build``. If
it is missing, loading raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnvfp4.so")
ABI_VERSION = 5

STATUS = {
    0: "NVFP4_SUCCESS",
    1: "NVFP4_ERROR_INVALID_VALUE",
    2: "NVFP4_ERROR_INVALID_SHAPE",
    3: "NVFP4_ERROR_MISALIGNED",
    4: "NVFP4_ERROR_WORKSPACE",
    5: "NVFP4_ERROR_UNSUPPORTED_DEVICE",
    6: "NVFP4_ERROR_HIP",
    7: "NVFP4_ERROR_TOO_LARGE",
}
SUCCESS, INVALID_VALUE, INVALID_SHAPE, MISALIGNED, WORKSPACE, UNSUPPORTED_DEVICE, HIP, TOO_LARGE = range(8)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_int = ctypes.c_int

# name -> (restype, argtypes); every function declared in include/*.h
SIGNATURES = {
    "nvfp4_abi_version": (_int, []),
    "nvfp4_status_string": (ctypes.c_char_p, [_int]),
    "nvfp4_last_hip_error": (_int, []),
    "nvfp4_quantize": (_int, [_vp, _i64, _i64, _f32, _vp, _vp, _vp]),
    "nvfp4_gemm": (_int, [_vp, _vp, _f32, _vp, _vp, _f32, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_gemm_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_int)]),
    "nvfp4_linear_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_int)]),
    "nvfp4_gemm_w4a16": (_int, [_vp, _vp, _vp, _f32, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_gemm_w4a16_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_int)]),
    "nvfp4_mxfp8_quantize": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "nvfp4_mxfp8_gemm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_mxfp8_quantize_elem": (_int, [_vp, _i64, _i64, _int, _vp, _vp, _vp]),
    "nvfp4_mxfp8_gemm_elem": (_int, [_vp, _vp, _int, _vp, _vp, _int, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_fp8r_quantize": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "nvfp4_fp8r_gemm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_linear_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "nvfp4_linear": (_int, [_vp, _f32, _vp, _vp, _f32, _i64, _i64, _i64, _vp, _vp,
                            ctypes.c_size_t, _vp]),
    "nvfp4_linear_noalloc": (_int, [_vp, _f32, _vp, _vp, _f32, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_amax": (_int, [_vp, _i64, _vp, _vp]),
    "nvfp4_global_scale_from_amax": (_f32, [_f32]),
    "nvfp4_calibrate_device": (_int, [_vp, _i64, _vp, _vp]),
    "nvfp4_quantize_devgs": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_gemm_devgs": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "nvfp4_linear_devgs": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp,
                                  ctypes.c_size_t, _vp]),
    "nvfp4_selftest_e2m1_encode": (_int, [_vp, _vp, _vp, _i64, _vp]),
    "nvfp4_selftest_e2m1_exhaustive": (_int, [_vp, _vp, _vp]),
    "nvfp4_selftest_division": (_int, [_vp, _vp, _vp]),
    "nvfp4_selftest_bf16_exhaustive": (_int, [_vp, _vp, _vp]),
    "nvfp4_selftest_mxfp8_e4m3_exhaustive": (_int, [_vp, _vp, _vp]),
    "nvfp4_selftest_mxfp8_e5m2_exhaustive": (_int, [_vp, _vp, _vp]),
    "nvfp4_selftest_block_scale": (_int, [_vp, _f32, _vp, _vp, _i64, _vp]),
    "nvfp4_selftest_decode": (_int, [_vp, _vp, _vp, _vp, _i64, _vp]),
}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        name = STATUS.get(status, f"status {status}")
        extra = f" (hipError {hip_error})" if status == HIP else ""
        super().__init__(f"{where}: {name}{extra}")


_lock = threading.Lock()
_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libnvfp4.so once and bind every entry point; raise if it is absent."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise FileNotFoundError(
                f"{p} is missing: build it with `python -m nvfp4_block_scaled_02_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        v = lib.nvfp4_abi_version()
        if v != ABI_VERSION:
            raise RuntimeError(f"libnvfp4 ABI version {v}, binding expects {ABI_VERSION}")
        if path is None:
            _lib = lib
        return lib


def check(status: int, where: str) -> None:
    if status != SUCCESS:
        hip = load_library().nvfp4_last_hip_error() if status == HIP else 0
        raise NVFP4Error(status, where, hip)
