"""Seeded synthetic inputs shaped like the linear layers of a FLUX-style transformer.

This package only draws random numbers and rounds them to bf16 storage; it holds none
of the NVFP4 arithmetic. Both the oracle side (tests) and the product side (tests,
bench) take their inputs from here.
"""
from .flux import WORKLOADS, Workload, make, names, to_bf16_bits  # noqa: F401
