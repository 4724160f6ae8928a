"""Seeded synthetic inputs for the FP8 grouped matmul workloads.

This module is shared by the tests, the smoke check and the benchmark.  It only
draws random numbers (expert routing counts and normally distributed bf16 tensors);
it holds none of the quantization or matmul arithmetic, and it imports neither the
CPU oracle nor the HIP library.

The workloads stand in for the MoE expert layers the pages discuss (DeepSeek-style
batch split, Mixtral-style merged gate|up): no dataset or trained weights are used.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    group_sizes_for,
    multinomial_sizes,
    normal_bf16,
    zipf_sizes,
)
