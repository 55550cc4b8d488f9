"""Python binding of libpa's host-side KV block manager (include/pa_blocks.h).

Argument marshalling only: the free-block queue, allocate_slots, per-block prefix
hashing and the step arrays all live in the library's C++ code. Runs on the host; no
GPU is needed.
"""

from __future__ import annotations

import ctypes
import sys

import numpy as np

from . import _lib
from .ops import PAError, _check

HASHES = {"fnv1a64": 0, "sha256": 1}
PA_E_NO_SPACE = 8


class NoSpace(PAError):
    """allocate_slots found too few free blocks; the manager is unchanged."""


def _i32(values) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


def _addr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def block_hash(tokens, parent: bytes | None = None, kind: str = "sha256") -> bytes:
    """The hash of one 16-token block under ``parent`` (32 bytes; None = zeros)."""
    lib = _lib.load()
    t = _i32(tokens)
    if t.shape != (_lib.BLOCK_SIZE,):
        raise ValueError("a block has 16 tokens")
    out = ctypes.create_string_buffer(32)
    par = ctypes.create_string_buffer(bytes(parent), 32) if parent is not None else None
    _check(lib.pa_block_hash_compute(HASHES[kind], par, _addr(t), out))
    return out.raw


class BlockManager:
    """A pool of ``num_blocks`` 16-token KV blocks handed out to requests.

    ``prefix_caching`` reuses full blocks whose chain hash is cached; ``hash`` is
    "fnv1a64" or "sha256".
    """

    def __init__(self, num_blocks: int, prefix_caching: bool = True, hash: str = "sha256"):
        self._lib = _lib.load()
        handle = ctypes.c_void_p(0)
        _check(self._lib.pa_bm_create(int(num_blocks), 1 if prefix_caching else 0, HASHES[hash],
                                      ctypes.byref(handle)))
        self._h = handle
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        if not sys.is_finalizing():
            self.close()

    def add_request(self, request_id: int, token_ids) -> int:
        """Register a request's prompt; returns the tokens served by the prefix cache."""
        t = _i32(token_ids)
        n = ctypes.c_int64(0)
        _check(self._lib.pa_bm_add_request(self._h, int(request_id), _addr(t), t.size, ctypes.byref(n)))
        return int(n.value)

    def append_tokens(self, request_id: int, token_ids) -> None:
        t = _i32(token_ids)
        _check(self._lib.pa_bm_append_tokens(self._h, int(request_id), _addr(t), t.size))

    def allocate_slots(self, request_id: int, num_new_tokens: int) -> None:
        """Make room for the next tokens; raises NoSpace (manager unchanged) if blocks run out."""
        status = self._lib.pa_bm_allocate_slots(self._h, int(request_id), int(num_new_tokens))
        if status == PA_E_NO_SPACE:
            raise NoSpace(status, self._lib.pa_last_error().decode(errors="replace"))
        _check(status)

    def free_request(self, request_id: int) -> None:
        _check(self._lib.pa_bm_free_request(self._h, int(request_id)))

    def build_step(self, request_ids, query_lens, max_blocks_per_seq: int, num_tokens: int | None = None):
        """Block tables, lengths, query offsets and slot mapping of one step (numpy, host)."""
        ids = np.ascontiguousarray(np.asarray(request_ids, dtype=np.int64))
        ql = np.ascontiguousarray(np.asarray(query_lens, dtype=np.int64))
        S = ids.size
        if ql.size != S:
            raise ValueError("request_ids and query_lens differ in length")
        T = int(ql.sum()) if num_tokens is None else int(num_tokens)
        bt = np.zeros((S, max_blocks_per_seq), dtype=np.int32)
        seq_lens = np.zeros(S, dtype=np.int32)
        ctx = np.zeros(S, dtype=np.int32)
        qsl = np.zeros(S + 1, dtype=np.int32)
        slots = np.zeros(max(T, 0), dtype=np.int64)
        _check(self._lib.pa_bm_build_step(self._h, _addr(ids), _addr(ql), S, int(max_blocks_per_seq), _addr(bt),
                                          _addr(seq_lens), _addr(qsl), _addr(ctx), _addr(slots), T))
        return {"block_tables": bt, "seq_lens": seq_lens, "query_start_loc": qsl, "context_lens": ctx,
                "slot_mapping": slots}

    @property
    def num_free_blocks(self) -> int:
        n = ctypes.c_int32(0)
        _check(self._lib.pa_bm_num_free_blocks(self._h, ctypes.byref(n)))
        return int(n.value)

    @property
    def num_cached_blocks(self) -> int:
        n = ctypes.c_int32(0)
        _check(self._lib.pa_bm_num_cached_blocks(self._h, ctypes.byref(n)))
        return int(n.value)

    def request_blocks(self, request_id: int) -> list[int]:
        n = ctypes.c_int32(0)
        _check(self._lib.pa_bm_request_blocks(self._h, int(request_id), None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), dtype=np.int32)
        _check(self._lib.pa_bm_request_blocks(self._h, int(request_id), _addr(out), out.size, ctypes.byref(n)))
        return out[: n.value].tolist()

    def request_info(self, request_id: int) -> dict:
        info = np.zeros(4, dtype=np.int64)
        _check(self._lib.pa_bm_request_info(self._h, int(request_id), _addr(info)))
        return {"known_tokens": int(info[0]), "computed_tokens": int(info[1]), "cache_hit_tokens": int(info[2]),
                "blocks": int(info[3])}

    def block_state(self, block: int) -> tuple[int, int]:
        """(reference count, position in the free queue or -1)."""
        ref, pos = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(self._lib.pa_bm_block_state(self._h, int(block), ctypes.byref(ref), ctypes.byref(pos)))
        return int(ref.value), int(pos.value)
