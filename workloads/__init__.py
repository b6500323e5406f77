"""Seeded synthetic inputs and exact work counters for packed variable-length attention.

This package holds no attention arithmetic.  It draws sequence lengths and
random tensors, rounds draws to bf16, builds the `cu_seqlens` boundaries of a
packed token stream, and counts visible (query, key) pairs.  Both the CPU
oracle's tests and the GPU path's tests, bench and smoke take their inputs
from here, so the two sides always see the same host arrays.
"""

from .generate import (  # noqa: F401
    Workload,
    bf16_bits,
    bf16_round,
    config,
    make_case,
    padding_mask,
    CONFIG_IDS,
)
from .count import (  # noqa: F401
    visible_pairs,
    workload_pairs,
    fwd_flops,
    bwd_flops,
    fwd_bytes,
    bwd_bytes,
)
