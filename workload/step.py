"""One synthetic step: lengths, block tables, block pool and new-token rows.

Pool layout (fixed by the library's C header and assumed by the oracle):

* ``k_cache[b, h, o, :]`` holds the key of the token stored at slot ``16*b + o``
  for kv head ``h``  -> shape ``[NB, Hkv, 16, D]``;
* ``v_cache[b, h, :, o]`` holds the value of that token     -> shape ``[NB, Hkv, D, 16]``.

Everything here is drawn from seeded generators: integer choices (lengths, block
permutations) from numpy's ``default_rng`` over a ``SeedSequence``, and the floating
point payload from a ``torch.Generator`` on the target device, so that multi-GB
pools are drawn at device speed.  Slots that hold no cached token (the tail of a
partially filled block, blocks no sequence owns, and the slots this step's new
tokens will be written to) are filled with NaN when ``poison`` is set, so a kernel
that reads a slot it must not read produces NaN instead of a plausible number.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 16

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Step:
    """All inputs of one paged-attention step (tensors live on one device)."""

    name: str
    dtype: str                      # "f32" or "bf16"
    q: torch.Tensor                 # [T, Hq, D]
    k: torch.Tensor                 # [T, Hkv, D]   new keys of this step
    v: torch.Tensor                 # [T, Hkv, D]   new values of this step
    k_cache: torch.Tensor           # [NB, Hkv, 16, D] before this step's tokens are written
    v_cache: torch.Tensor           # [NB, Hkv, D, 16]
    block_tables: torch.Tensor      # int32 [S, MB], unused entries are -1
    seq_lens: torch.Tensor          # int32 [S]  tokens after this step (context + new)
    query_start_loc: torch.Tensor   # int32 [S+1]
    context_lens: torch.Tensor      # int32 [S]  tokens cached before this step
    scale: float
    meta: dict = field(default_factory=dict)

    # -- sizes -------------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def device(self) -> torch.device:
        return self.q.device

    def to(self, device) -> "Step":
        moved = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for key, val in moved.items():
            if isinstance(val, torch.Tensor):
                moved[key] = val.to(device)
        moved["meta"] = dict(self.meta)
        return Step(**moved)

    def clone(self) -> "Step":
        copied = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for key, val in copied.items():
            if isinstance(val, torch.Tensor):
                copied[key] = val.clone()
        copied["meta"] = dict(self.meta)
        return Step(**copied)

    def lengths(self):
        """Host copies of (context_lens, query lengths, seq_lens) as int64 numpy arrays."""
        ctx = self.context_lens.cpu().numpy().astype(np.int64)
        qsl = self.query_start_loc.cpu().numpy().astype(np.int64)
        return ctx, np.diff(qsl), self.seq_lens.cpu().numpy().astype(np.int64)


def _rngs(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _torch_gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    gen = torch.Generator(device=dev) if dev.type != "cpu" else torch.Generator()
    gen.manual_seed(int(np.random.SeedSequence([seed, 0x5EED]).generate_state(1)[0]))
    return gen


def _normal(shape, dtype: str, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=_TORCH_DTYPES[dtype])


def build_step(
    context_lens: Sequence[int],
    query_lens: Sequence[int],
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str,
    scale: Optional[float] = None,
    num_blocks: Optional[int] = None,
    max_blocks_per_seq: Optional[int] = None,
    shared_prefix_tokens: int = 0,
    seed: int = 0,
    device="cpu",
    poison: bool = True,
    name: str = "custom",
) -> Step:
    """Draw one step for the given per-sequence context and query lengths.

    Physical block ids come from one seeded permutation of ``range(num_blocks)``,
    dealt out in sequence order (after ``shared_prefix_tokens // 16`` ids that every
    sequence lists first, when a shared prefix is asked for).
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    qlen = np.asarray(query_lens, dtype=np.int64)
    if ctx.shape != qlen.shape or ctx.ndim != 1:
        raise ValueError("context_lens and query_lens must be 1-D and of equal length")
    if (ctx < 0).any() or (qlen < 0).any():
        raise ValueError("lengths must be non-negative")
    if dtype not in _TORCH_DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_TORCH_DTYPES)}")
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    S = int(ctx.shape[0])
    L = ctx + qlen
    nblk = (L + BLOCK_SIZE - 1) // BLOCK_SIZE
    if shared_prefix_tokens % BLOCK_SIZE:
        raise ValueError("a shared prefix must be a whole number of blocks")
    n_shared = shared_prefix_tokens // BLOCK_SIZE
    if n_shared and (ctx < shared_prefix_tokens).any():
        raise ValueError("every sequence must hold the whole shared prefix in its context")
    needed = n_shared + int(np.maximum(nblk - n_shared, 0).sum())
    if num_blocks is None:
        num_blocks = max(needed, 1)
    if num_blocks < needed:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold the {needed} blocks needed")
    mb = int(nblk.max()) if S else 1
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(mb, 1)
    if max_blocks_per_seq < mb:
        raise ValueError("max_blocks_per_seq is smaller than the longest sequence needs")

    rng_blocks, = _rngs(seed, 1)
    order = rng_blocks.permutation(num_blocks).astype(np.int64)
    tables = np.full((S, max_blocks_per_seq), -1, dtype=np.int32)
    shared_ids = order[:n_shared]
    cursor = n_shared
    for i in range(S):
        tables[i, :n_shared] = shared_ids
        own = int(nblk[i]) - n_shared
        tables[i, n_shared:n_shared + own] = order[cursor:cursor + own]
        cursor += own

    # Which slots of each physical block hold a cached (pre-step) token.
    filled = np.zeros(num_blocks, dtype=np.int64)
    for i in range(S):
        for b in range(int(nblk[i])):
            count = int(min(max(ctx[i] - BLOCK_SIZE * b, 0), BLOCK_SIZE))
            phys = int(tables[i, b])
            filled[phys] = max(filled[phys], count)

    dev = torch.device(device)
    gen = _torch_gen(seed, dev)
    T = int(qlen.sum())
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    k_cache = _normal((num_blocks, Hkv, BLOCK_SIZE, D), dtype, gen, dev)
    v_cache = _normal((num_blocks, Hkv, D, BLOCK_SIZE), dtype, gen, dev)
    q = _normal((T, Hq, D), dtype, gen, dev)
    k = _normal((T, Hkv, D), dtype, gen, dev)
    v = _normal((T, Hkv, D), dtype, gen, dev)
    if poison:
        live = torch.arange(BLOCK_SIZE, device=dev)[None, :] < torch.from_numpy(filled).to(dev)[:, None]
        k_cache.masked_fill_(~live[:, None, :, None], float("nan"))
        v_cache.masked_fill_(~live[:, None, None, :], float("nan"))

    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(qlen)
    if scale is None:
        scale = 1.0 / float(np.sqrt(head_dim))
    as_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return Step(
        name=name,
        dtype=dtype,
        q=q,
        k=k,
        v=v,
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=as_dev(tables),
        seq_lens=as_dev(L.astype(np.int32)),
        query_start_loc=as_dev(qsl),
        context_lens=as_dev(ctx.astype(np.int32)),
        scale=float(scale),
        meta={"seed": seed, "shared_prefix_tokens": shared_prefix_tokens, "poison": poison},
    )


# ---------------------------------------------------------------------------
# Input transformations used by the invariance tests.  Each returns a new Step
# whose logical content (every sequence's tokens in logical order) is unchanged.
# ---------------------------------------------------------------------------

def permute_blocks(step: Step, seed: int) -> Step:
    """Relabel physical blocks: block ``b`` moves to ``perm[b]`` and the tables follow."""
    rng, = _rngs(seed, 1)
    nb = step.num_blocks
    perm = torch.from_numpy(rng.permutation(nb).astype(np.int64)).to(step.device)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(nb, device=step.device)
    out = step.clone()
    out.k_cache = step.k_cache[inv]
    out.v_cache = step.v_cache[inv]
    bt = step.block_tables.long()
    mapped = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt)
    out.block_tables = mapped.to(torch.int32)
    out.meta["permuted_with"] = seed
    return out


def privatize_shared_prefix(step: Step, seed: int = 0) -> Step:
    """Give every sequence its own copy of the shared prefix blocks (same data, new ids)."""
    n_shared = step.meta.get("shared_prefix_tokens", 0) // BLOCK_SIZE
    if n_shared == 0:
        raise ValueError("step has no shared prefix")
    S, nb = step.num_seqs, step.num_blocks
    rng, = _rngs(seed, 1)
    # Copy r = i*n_shared + j (sequence i, prefix block j) lands in pool row nb + perm[r].
    perm = torch.from_numpy(rng.permutation(S * n_shared).astype(np.int64)).to(step.device)
    shared = step.block_tables[0, :n_shared].long()
    src = shared.repeat(S)
    extra_k = torch.empty((S * n_shared,) + tuple(step.k_cache.shape[1:]), dtype=step.k_cache.dtype, device=step.device)
    extra_v = torch.empty((S * n_shared,) + tuple(step.v_cache.shape[1:]), dtype=step.v_cache.dtype, device=step.device)
    extra_k[perm] = step.k_cache[src]
    extra_v[perm] = step.v_cache[src]
    out = step.clone()
    out.k_cache = torch.cat([step.k_cache, extra_k], dim=0)
    out.v_cache = torch.cat([step.v_cache, extra_v], dim=0)
    bt = step.block_tables.clone()
    bt[:, :n_shared] = (nb + perm.view(S, n_shared)).to(torch.int32)
    out.block_tables = bt
    out.meta["shared_prefix_tokens"] = 0
    out.meta["privatized_prefix_blocks"] = n_shared
    return out


def shuffle_sequences(step: Step, seed: int) -> Step:
    """Reorder the sequences of the step (rows of q/k/v move with their sequence)."""
    rng, = _rngs(seed, 1)
    S = step.num_seqs
    perm = rng.permutation(S)
    return subset_sequences(step, perm, compact_pool=False)


def subset_sequences(step: Step, seqs, compact_pool: bool = True) -> Step:
    """A step holding only ``seqs`` (in that order).

    With ``compact_pool`` the pool shrinks to the blocks these sequences list, in
    first-use order; otherwise the pool is shared with ``step`` unchanged.
    """
    seqs = np.asarray(seqs, dtype=np.int64)
    ctx, qlen, L = step.lengths()
    qsl = step.query_start_loc.cpu().numpy().astype(np.int64)
    rows = np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in seqs]) if len(seqs) else np.zeros(0, np.int64)
    rows_t = torch.from_numpy(rows).to(step.device)
    bt = step.block_tables[torch.from_numpy(seqs).to(step.device)].clone()
    out = step.clone()
    out.q, out.k, out.v = step.q[rows_t], step.k[rows_t], step.v[rows_t]
    if compact_pool:
        bt_host = bt.cpu().numpy()
        used = []
        seen = {}
        nblk = (L[seqs] + BLOCK_SIZE - 1) // BLOCK_SIZE
        for r in range(len(seqs)):
            for b in range(int(nblk[r])):
                phys = int(bt_host[r, b])
                if phys not in seen:
                    seen[phys] = len(used)
                    used.append(phys)
        remap = np.full(step.num_blocks, -1, dtype=np.int64)
        remap[np.asarray(used, dtype=np.int64)] = np.arange(len(used))
        new_bt = np.full_like(bt_host, -1)
        for r in range(len(seqs)):
            new_bt[r, : int(nblk[r])] = remap[bt_host[r, : int(nblk[r])]]
        idx = torch.from_numpy(np.asarray(used, dtype=np.int64)).to(step.device)
        out.k_cache = step.k_cache[idx] if len(used) else step.k_cache[:1].clone()
        out.v_cache = step.v_cache[idx] if len(used) else step.v_cache[:1].clone()
        bt = torch.from_numpy(new_bt).to(step.device)
    out.block_tables = bt
    out.seq_lens = step.seq_lens[torch.from_numpy(seqs).to(step.device)].clone()
    out.context_lens = step.context_lens[torch.from_numpy(seqs).to(step.device)].clone()
    new_qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
    new_qsl[1:] = np.cumsum(qlen[seqs])
    out.query_start_loc = torch.from_numpy(new_qsl).to(step.device)
    out.meta["subset_of"] = step.name
    return out


def random_slots(num_tokens: int, num_blocks: int, *, pad_fraction: float = 0.0, seed: int = 0) -> np.ndarray:
    """Distinct random cache slots in ``[0, 16*num_blocks)``; a fraction are ``-1`` (skip)."""
    if num_tokens > num_blocks * BLOCK_SIZE:
        raise ValueError("more tokens than slots")
    rng_slots, rng_pad = _rngs(seed, 2)
    slots = rng_slots.choice(num_blocks * BLOCK_SIZE, size=num_tokens, replace=False).astype(np.int64)
    if pad_fraction > 0:
        slots[rng_pad.random(num_tokens) < pad_fraction] = -1
    return slots


def host_arrays(step: Step) -> dict:
    """Host numpy copies of a step's arrays, as the oracle takes them.

    fp32 payloads stay ``float32``; bf16 payloads become ``uint16`` arrays of the raw
    bfloat16 bit patterns (numpy has no bfloat16 type).
    """
    def payload(t: torch.Tensor) -> np.ndarray:
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float32:
            return t.numpy()
        raise TypeError(f"unexpected payload dtype {t.dtype}")

    return {
        "q": payload(step.q),
        "k": payload(step.k),
        "v": payload(step.v),
        "k_cache": payload(step.k_cache),
        "v_cache": payload(step.v_cache),
        "block_tables": step.block_tables.cpu().numpy().astype(np.int64),
        "seq_lens": step.seq_lens.cpu().numpy().astype(np.int64),
        "query_start_loc": step.query_start_loc.cpu().numpy().astype(np.int64),
        "context_lens": step.context_lens.cpu().numpy().astype(np.int64),
        "scale": step.scale,
    }
