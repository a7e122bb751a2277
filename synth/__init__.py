"""Seeded synthetic workloads for the MiniMax-M3 pre-attention prologue and the
DSpark drafter's attention.

This module only draws random inputs (activations, gammas, weights, RoPE table,
positions, slot mappings, sentinel-filled caches). It holds none of the
prologue's arithmetic: number-format conversions of the random draws go through
torch's own casts. Both the oracle tests and the GPU path take their inputs
from here.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    SENTINEL_CACHE_BYTE,
    SENTINEL_SCALE_BITS,
    Workload,
    make_workload,
    named_config,
    with_nvfp4_caches,
)
from .drafter import make_drafter  # noqa: F401,E402
