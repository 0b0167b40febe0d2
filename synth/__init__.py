"""Seeded synthetic inputs for paged MLA decode.

This package only draws random numbers and lays them out (query bits, latent
rows, lengths, page maps).  It holds none of the attention or quantisation
arithmetic, so both the HIP path and the CPU oracle can take their inputs
from it without sharing any of the method.
"""

from .workloads import (  # noqa: F401
    D,
    DV,
    PAGE,
    SOFTMAX_SCALE,
    Workload,
    bf16_bits,
    custom,
    make,
    CONFIG_NAMES,
    EXTEND_NAMES,
)
