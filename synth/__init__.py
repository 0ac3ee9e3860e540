"""Seeded synthetic inputs for the BDLM attention workloads.

This package holds random draws, their scaling and dtype casts, and the shape
tables of the workloads.  It holds none of the attention arithmetic, so both the
oracle-side tests and the GPU-side calls can take their inputs from it.
"""
from .inputs import (  # noqa: F401
    TENSOR_ORDER,
    draw_normal,
    make_full_inputs,
    make_share_inputs,
    clean_shard_ids,
    draw_block_positions,
    draw_units,
    to_f64,
)
from .workloads import WORKLOADS, Workload  # noqa: F401
