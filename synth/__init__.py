"""Seeded synthetic workloads for the NVFP4 W4A4 + residual-compensation path.

This package only draws random inputs (bf16 bit patterns, float32 router
logits) with the shapes and value distributions of the five workloads; it
contains none of the method's arithmetic.  The tests and the benchmark feed
the same host arrays to both the HIP library and the CPU oracle.
"""
from .configs import CONFIGS, Config, get  # noqa: F401
from .gen import Workload, make  # noqa: F401
