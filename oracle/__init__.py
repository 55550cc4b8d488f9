"""CPU oracle for one paged-attention step, and a model of the host-side KV block
manager (``block_manager``) -- TEST INFRASTRUCTURE, not product code.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``paged_kv_cache_460_amd``) and imports nothing from it.
"""

from . import block_manager
from .paged_attention import (
    BLOCK_SIZE,
    OracleInputError,
    attention,
    gather_sequence,
    reshape_and_cache,
    slot_mapping,
    validate_step,
    widen,
)

__all__ = [
    "BLOCK_SIZE",
    "block_manager",
    "OracleInputError",
    "attention",
    "gather_sequence",
    "reshape_and_cache",
    "slot_mapping",
    "validate_step",
    "widen",
]
