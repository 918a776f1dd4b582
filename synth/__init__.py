"""Seeded synthetic inputs shared by the tests, the oracle checks and bench.py.

This package only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, quantization, placement or attention).
"""

from .workloads import CONFIGS, Workload, get, bf16_from_f32  # noqa: F401
