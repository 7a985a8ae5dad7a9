"""Seeded synthetic inputs for the routed MoE expert layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds the five workload shapes and the recipe that turns a seed
into tensors; it holds none of the layer's own arithmetic (no alignment, no
GEMM, no activation, no combine).  Routing (logits -> softmax -> top-k) and the
weight block quantisation of the fp8 workload live here because they produce
the layer's *inputs*: the layer receives expert ids, routing weights and
already-quantised weights.
"""
from .configs import CONFIGS, SWEEP_CONFIGS, MoEConfig, get_config, sweep_batch_sizes  # noqa: F401
from .generate import (  # noqa: F401
    MoECase,
    MXCase,
    make_case,
    make_mx_case,
    mx_quantize,
    make_logits,
    make_routing,
    make_x,
    routing_stats,
    slab_seed,
)
