"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This package holds no arithmetic of the dispatch/combine method: it only draws
routing tables, routing weights and activations.  Both the CPU oracle and the
HIP path receive the very same arrays from here.
"""

from .workloads import (  # noqa: F401
    CONFIG_ORDER,
    CONFIGS,
    Workload,
    by_index,
    gen_bf16_rows,
    gen_cached_x,
    gen_expert_out,
    gen_grad_out,
    gen_routing,
    gen_weights,
    gen_x,
    scaled,
)
