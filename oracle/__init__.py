"""CPU oracle for the NVFP4 W4A4 linear path -- test infrastructure, not product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library: no
kernels, headers, tables, constants generators or pre/post-processing.

* ``oracle.nvfp4_oracle``  -- vectorised NumPy oracle (quantize, dequantize, GEMM
  reference in float64, exact int64 GEMM, tolerance check).
* ``oracle.scalar_oracle`` -- exact ``Fraction`` brute force used to pin the former.
"""
from . import nvfp4_oracle, scalar_oracle  # noqa: F401
