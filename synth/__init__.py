"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package draws random numbers and names workload shapes. It holds none of
the method's arithmetic: no quantization, no dot products, no dequantization.
"""
from .inputs import *  # noqa: F401,F403
