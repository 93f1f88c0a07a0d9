"""Seeded synthetic inputs for the per-round verify-and-route step.

This package draws random numbers and lays them out; it holds none of the
method's arithmetic (no argmax, no acceptance rule, no router).  Both the HIP
path and the CPU oracle consume what it produces.
"""

from .workloads import (  # noqa: F401
    V_QWEN3,
    D_QWEN3,
    VD_EAGLE3,
    CONFIGS,
    ChainBatch,
    TreeBatch,
    RouterInputs,
    RoutedBatch,
    f32_to_bf16_bits,
    make_chain_batch,
    make_tree_batch,
    make_router_inputs,
    negate_second_layer,
    make_routed_batch,
    make_d2t,
    make_config,
    routed_calibration,
    make_hidden_rows,
)
