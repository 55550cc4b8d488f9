"""Python binding over libpa's C entry points.

Argument marshalling only: torch supplies device memory and the current HIP stream;
every step of the computation runs in the library's kernels. There is no fallback
path: if libpa.so is missing, or a tensor is not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import sys

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.PA_F32, torch.bfloat16: _lib.PA_BF16}


class PAError(RuntimeError):
    """A libpa call returned a non-OK status."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = _lib.STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def _check(status: int) -> None:
    if status != 0:
        detail = _lib.load().pa_last_error().decode(errors="replace")
        raise PAError(status, detail)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device}); libpa has no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _payload_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} must be float32 or bfloat16 (got {t.dtype})")
    return _DTYPES[t.dtype]


def build_slot_mapping(block_tables, query_start_loc, context_lens, num_tokens=None, with_positions=True):
    """Positions ([T] int32) and slot mapping ([T] int64) of the step's tokens.

    ``num_tokens`` defaults to ``query_start_loc[-1]`` (read from the device).
    """
    lib = _lib.load()
    dev = block_tables.device
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    S, MB = block_tables.shape
    if query_start_loc.shape[0] != S + 1 or context_lens.shape[0] != S:
        raise ValueError("query_start_loc must be [S+1] and context_lens [S]")
    if num_tokens is None:
        num_tokens = int(query_start_loc[-1].item())
    slots = torch.empty(num_tokens, dtype=torch.int64, device=dev)
    positions = torch.empty(num_tokens, dtype=torch.int32, device=dev) if with_positions else None
    _check(lib.pa_build_slot_mapping(_ptr(block_tables), _ptr(query_start_loc), _ptr(context_lens), S, MB,
                                     num_tokens, _ptr(positions), _ptr(slots), _stream(block_tables)))
    return positions, slots


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping) -> None:
    """Write the step's new K/V rows into the block pool at their slots (in place)."""
    lib = _lib.load()
    dev = k.device
    _need(k, "k", ndim=3)
    dt = _payload_dtype(k, "k")
    _need(v, "v", k.dtype, 3, dev)
    _need(k_cache, "k_cache", k.dtype, 4, dev)
    _need(v_cache, "v_cache", k.dtype, 4, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    T, hkv, d = k.shape
    nb = k_cache.shape[0]
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape [T, Hkv, D]")
    if tuple(k_cache.shape) != (nb, hkv, _lib.BLOCK_SIZE, d) or tuple(v_cache.shape) != (nb, hkv, d, _lib.BLOCK_SIZE):
        raise ValueError("caches must be [NB, Hkv, 16, D] (keys) and [NB, Hkv, D, 16] (values)")
    if slot_mapping.shape[0] < T:
        raise ValueError("slot_mapping shorter than the number of tokens")
    _check(lib.pa_reshape_and_cache(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, hkv,
                                    d, nb, dt, _stream(k)))


def attention_workspace_size(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads, head_dim,
                             dtype) -> int:
    lib = _lib.load()
    out = ctypes.c_size_t(0)
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    _check(lib.pa_attention_workspace_size(num_seqs, max_blocks_per_seq, num_tokens, num_q_heads, num_kv_heads,
                                           head_dim, dt, ctypes.byref(out)))
    return int(out.value)


def attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out=None,
              workspace=None):
    """Attention over one mixed step; returns ``out`` ([T, Hq, D], q's dtype).

    The caches must already hold this step's tokens (``reshape_and_cache`` first).
    ``workspace`` (optional) is a uint8 device tensor of at least
    ``attention_workspace_size(...)`` bytes; one is allocated when it is omitted.
    """
    lib = _lib.load()
    dev = q.device
    _need(q, "q", ndim=3)
    dt = _payload_dtype(q, "q")
    _need(k_cache, "k_cache", q.dtype, 4, dev)
    _need(v_cache, "v_cache", q.dtype, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    _need(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    T, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    S, MB = block_tables.shape
    if tuple(k_cache.shape) != (nb, hkv, _lib.BLOCK_SIZE, d) or tuple(v_cache.shape) != (nb, hkv, d, _lib.BLOCK_SIZE):
        raise ValueError("caches must be [NB, Hkv, 16, D] (keys) and [NB, Hkv, D, 16] (values)")
    if seq_lens.shape[0] != S or context_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens/context_lens must be [S] and query_start_loc [S+1]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype, 3, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need = attention_workspace_size(S, MB, T, hq, hkv, d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    _check(lib.pa_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
                            _ptr(query_start_loc), _ptr(context_lens), float(scale), _ptr(out), S, MB, T, hq, hkv,
                            d, nb, dt, _ptr(workspace), workspace.numel(), _stream(q)))
    return out


def attention_noalloc(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out):
    """``attention`` into a caller-provided ``out`` with the library's fixed scratch as the
    workspace (pa_attention_noalloc in pa.h): the library allocates nothing. Sizes needing
    more than ``NOALLOC_SCRATCH_BYTES`` of workspace raise PAError (PA_E_WORKSPACE)."""
    lib = _lib.load()
    dev = q.device
    _need(q, "q", ndim=3)
    dt = _payload_dtype(q, "q")
    _need(k_cache, "k_cache", q.dtype, 4, dev)
    _need(v_cache, "v_cache", q.dtype, 4, dev)
    _need(block_tables, "block_tables", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    _need(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    _need(out, "out", q.dtype, 3, dev)
    T, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    S, MB = block_tables.shape
    if tuple(k_cache.shape) != (nb, hkv, _lib.BLOCK_SIZE, d) or tuple(v_cache.shape) != (nb, hkv, d, _lib.BLOCK_SIZE):
        raise ValueError("caches must be [NB, Hkv, 16, D] (keys) and [NB, Hkv, D, 16] (values)")
    if seq_lens.shape[0] != S or context_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("seq_lens/context_lens must be [S] and query_start_loc [S+1]")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check(lib.pa_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
                                    _ptr(query_start_loc), _ptr(context_lens), float(scale), _ptr(out), S, MB, T,
                                    hq, hkv, d, nb, dt, _stream(q)))
    return out


def attention_plan_info(workspace, q, k_cache, block_tables):
    """The on-device planner's summary of the last ``attention`` call that used
    ``workspace`` with these tensors' sizes (see pa_attention_plan_info in pa.h)."""
    lib = _lib.load()
    _need(workspace, "workspace", torch.uint8, 1)
    T, hq, d = q.shape
    hkv = k_cache.shape[1]
    S, MB = block_tables.shape
    info = (ctypes.c_int32 * 7)()
    _check(lib.pa_attention_plan_info(_ptr(workspace), workspace.numel(), S, MB, T, hq, hkv, d,
                                      _payload_dtype(q, "q"), info, _stream(q)))
    return {"decode_tasks": info[0], "decode_rows": info[1], "shared_prefix_keys": info[2],
            "shared_prefix_parts": info[3], "partial_slots": info[4], "shared_prefix_part_keys": info[5],
            "partition_tokens": info[6]}


def step(q, k, v, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out=None,
         workspace=None, slot_mapping=None):
    """One whole step on the current stream: slot mapping, cache write, attention."""
    if slot_mapping is None:
        _, slot_mapping = build_slot_mapping(block_tables, query_start_loc, context_lens, num_tokens=q.shape[0],
                                             with_positions=False)
    reshape_and_cache(k, v, k_cache, v_cache, slot_mapping)
    return attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out=out,
                     workspace=workspace)


class StepGraph:
    """One step (slot mapping, cache write, attention) recorded as a HIP graph over fixed
    buffers and replayed with one launch (pa_step_graph_create in pa.h).

    Refill the input tensors in place between replays; the graph keeps their addresses
    and sizes. ``out``, ``slot_mapping`` ([T] int64), ``workspace`` and ``positions``
    ([T] int32, optional) are written by every replay. The tensors are kept alive for the
    graph's lifetime.
    """

    def __init__(self, q, k, v, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out,
                 slot_mapping, workspace, positions=None):
        lib = _lib.load()
        dev = q.device
        _need(q, "q", ndim=3)
        dt = _payload_dtype(q, "q")
        for t, name in ((k, "k"), (v, "v"), (out, "out")):
            _need(t, name, q.dtype, 3, dev)
        _need(k_cache, "k_cache", q.dtype, 4, dev)
        _need(v_cache, "v_cache", q.dtype, 4, dev)
        _need(block_tables, "block_tables", torch.int32, 2, dev)
        for t, name in ((seq_lens, "seq_lens"), (query_start_loc, "query_start_loc"), (context_lens, "context_lens")):
            _need(t, name, torch.int32, 1, dev)
        _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
        _need(workspace, "workspace", torch.uint8, 1, dev)
        if positions is not None:
            _need(positions, "positions", torch.int32, 1, dev)
        T, hq, d = q.shape
        nb, hkv = k_cache.shape[0], k_cache.shape[1]
        S, MB = block_tables.shape
        if k.shape != (T, hkv, d) or v.shape != k.shape or out.shape != q.shape:
            raise ValueError("k, v must be [T, Hkv, D] and out [T, Hq, D]")
        if tuple(k_cache.shape) != (nb, hkv, _lib.BLOCK_SIZE, d) or tuple(v_cache.shape) != (nb, hkv, d, _lib.BLOCK_SIZE):
            raise ValueError("caches must be [NB, Hkv, 16, D] (keys) and [NB, Hkv, D, 16] (values)")
        if seq_lens.shape[0] != S or context_lens.shape[0] != S or query_start_loc.shape[0] != S + 1:
            raise ValueError("seq_lens/context_lens must be [S] and query_start_loc [S+1]")
        if slot_mapping.shape[0] < T or (positions is not None and positions.shape[0] < T):
            raise ValueError("slot_mapping and positions need at least T entries")
        self._keep = (q, k, v, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, out,
                      slot_mapping, workspace, positions)
        self._device = dev
        self._lib = lib
        handle = ctypes.c_void_p(0)
        _check(lib.pa_step_graph_create(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                        _ptr(seq_lens), _ptr(query_start_loc), _ptr(context_lens), float(scale),
                                        _ptr(out), _ptr(positions), _ptr(slot_mapping), S, MB, T, hq, hkv, d, nb, dt,
                                        _ptr(workspace), workspace.numel(), ctypes.byref(handle)))
        self._handle = handle

    def replay(self) -> None:
        """Launch the recorded step on the current stream."""
        if not self._handle:
            raise RuntimeError("StepGraph is closed")
        stream = ctypes.c_void_p(torch.cuda.current_stream(self._device).cuda_stream)
        _check(self._lib.pa_step_graph_launch(self._handle, stream))

    def close(self) -> None:
        if getattr(self, "_handle", None):
            _check(self._lib.pa_step_graph_destroy(self._handle))
            self._handle = None
            self._keep = None

    def __del__(self):
        # At interpreter exit the HIP runtime may already be gone (and this module's
        # globals cleared): leave the graph to the OS.
        try:
            if sys.is_finalizing():
                return
        except Exception:
            return
        try:
            self.close()
        except Exception:
            pass


class KernelTimer:
    """Per-kernel GPU time recorded by libpa's event brackets (see pa_timing_* in pa.h)."""

    def __enter__(self):
        lib = _lib.load()
        _check(lib.pa_timing_reset())
        _check(lib.pa_timing_enable(1))
        return self

    def __exit__(self, *exc):
        _check(_lib.load().pa_timing_enable(0))
        return False

    @staticmethod
    def read(kind: str):
        """(total milliseconds, launches) for a kernel kind since the timer was entered."""
        lib = _lib.load()
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        _check(lib.pa_timing_read(_lib.KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(n)))
        return float(ms.value), int(n.value)
