"""Seeded synthetic inputs for the routed-expert FP8 MoE layer.

This package holds the workload table and the random-input generators that
both sides of every parity check draw from (the GPU library's tests and bench,
and the CPU oracle).  It contains none of the method's arithmetic: no
quantisation, routing, permutation or GEMM -- only shapes and random numbers.
"""

from .configs import CONFIGS, get_config
from .gen import tensor_seed, randn, layer_inputs, expert_weights, zipf_offsets, output_grad, router_weight

__all__ = ["CONFIGS", "get_config", "tensor_seed", "randn", "layer_inputs",
           "expert_weights", "zipf_offsets", "output_grad", "router_weight"]
