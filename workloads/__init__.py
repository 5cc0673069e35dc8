"""Seeded synthetic decode workloads shared by the oracle side and the GPU side.

This package only draws random numbers and lays them out: sequence lengths,
block tables, and bf16 queries / keys / values.  It holds none of the
method's arithmetic (no rotation, no quantization, no attention), so that the
oracle and the HIP path can both consume the same inputs without sharing any
code that computes the method.
"""

from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    Workload,
    build_workload,
    seq_kv,
    seq_query,
    chunk_queries,
    bf16_bits,
)
