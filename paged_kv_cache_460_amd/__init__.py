"""PagedAttention over a block-paged KV cache for AMD MI355X (gfx950).

The computation lives in ``libpa.so`` (C ABI in ``include/pa.h``, HIP kernels in
``csrc/``). This package is its Python binding.
"""

from ._lib import BLOCK_SIZE, LibraryMissing, LIB_PATH, load as load_library
from .blocks import BlockManager, NoSpace, block_hash
from .ops import (
    KernelTimer,
    PAError,
    StepGraph,
    attention,
    attention_noalloc,
    attention_plan_info,
    attention_workspace_size,
    build_slot_mapping,
    reshape_and_cache,
    step,
)

__all__ = [
    "BLOCK_SIZE",
    "BlockManager",
    "NoSpace",
    "block_hash",
    "KernelTimer",
    "LIB_PATH",
    "LibraryMissing",
    "PAError",
    "StepGraph",
    "attention",
    "attention_noalloc",
    "attention_plan_info",
    "attention_workspace_size",
    "build_slot_mapping",
    "load_library",
    "reshape_and_cache",
    "step",
]
