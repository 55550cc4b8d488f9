"""Seeded synthetic inputs for one paged-attention step.

This package only draws inputs: sequence lengths, the physical block assignment,
the block pool's contents and each new token's q/k/v rows.  It computes nothing of
the attention method itself (no slot mapping, no cache scatter, no softmax).  The
library's GPU tests, the CPU oracle's tests and ``bench.py`` all take their inputs
from here, so the two sides of every parity check see the same numbers.
"""

from .step import (
    BLOCK_SIZE,
    Step,
    build_step,
    host_arrays,
    permute_blocks,
    privatize_shared_prefix,
    random_slots,
    shuffle_sequences,
    subset_sequences,
)
from .configs import CONFIGS, make_config

__all__ = [
    "BLOCK_SIZE",
    "CONFIGS",
    "Step",
    "build_step",
    "host_arrays",
    "make_config",
    "permute_blocks",
    "privatize_shared_prefix",
    "random_slots",
    "shuffle_sequences",
    "subset_sequences",
]
