"""Seeded synthetic workloads for the packed DiT block.

This package only *generates inputs*: block shapes, packed layouts (token
positions and per-token modulation rows) and seeded random tensors.  It holds
none of the block's arithmetic, so both the CPU oracle and the HIP path can
draw from it without sharing any computation.
"""

from .workloads import (  # noqa: F401
    SPECS,
    BlockSpec,
    Workload,
    bf16_bits,
    bf16_round,
    build_layout,
    make_workload,
    spec_by_name,
)
