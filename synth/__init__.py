"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package draws random numbers and lays them out in the paged formats the
attention library reads. It holds none of the attention arithmetic: no dot
products, no softmax, no dequantisation, no page regeneration.
"""

from .workloads import (  # noqa: F401
    DTYPES,
    TIER_HOT,
    TIER_I8,
    TIER_I4,
    TIER_SHIFT,
    SLOT_MASK,
    Paged,
    build,
    config,
    CONFIG_SPECS,
)
