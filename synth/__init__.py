"""Seeded synthetic inputs shared by the oracle's tests and the GPU path's tests and bench."""
from .workloads import (WORKLOADS, Workload, capacity_for, f32_to_bf16_bits, load_params,
                        make_expert_bank, make_inputs, make_router, make_x)

__all__ = ["WORKLOADS", "Workload", "capacity_for", "f32_to_bf16_bits", "load_params",
           "make_expert_bank", "make_inputs", "make_router", "make_x"]
