"""Seeded synthetic inputs shared by the CPU oracle's tests, the GPU parity tests and the bench.

This package draws random numbers and rounds them to the storage dtype; it holds none of the
attention method's arithmetic. Both sides of every parity check receive the same tensors from here.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    gen_fp8_workload,
    gen_qkv,
    gen_qkv_device,
    gen_signs,
    normal_f32,
    workload,
)
