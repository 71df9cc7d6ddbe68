"""Seeded synthetic workloads for the paged-KV mixed step.

This module only draws data: sequence lengths, slot ids, the initial order of
the free block list, and the K/V/Q values.  It holds none of the method's
arithmetic (no block tables, no slot mappings, no attention).  Both the GPU
path and the CPU oracle consume exactly the bits produced here.
"""
from .configs import (  # noqa: F401
    CONFIG_NAMES,
    Segment,
    Step,
    Workload,
    bf16_bits_from_f32,
    make_prefix_share,
    make_workload,
    make_custom,
)
