"""CPU oracle for the NVFP4 W4A4 linear path (and the MXFP8 and fp8r paths) -- test
infrastructure, not product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library: no
kernels, headers, tables, constants generators or pre/post-processing.

* ``oracle.nvfp4_oracle``  -- vectorised NumPy oracle (quantize, dequantize, GEMM
  reference in float64, exact int64 GEMM, tolerance check).
* ``oracle.scalar_oracle`` -- exact ``Fraction`` brute force used to pin the former.
* ``oracle.mxfp8_oracle``  -- MXFP8 (OCP microscaling, E4M3 elements, 32-element
  blocks, E8M0 scales) quantize, dequantize and GEMM reference.
* ``oracle.fp8r_oracle``   -- rowwise FP8 (E4M3 elements, one fp32 scale per row)
  quantize, dequantize and GEMM reference.
"""
from . import fp8r_oracle, mxfp8_oracle, nvfp4_oracle, scalar_oracle  # noqa: F401
