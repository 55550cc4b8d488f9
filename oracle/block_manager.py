"""Plain-Python model of the host-side KV block manager -- TEST INFRASTRUCTURE.

Only the tests may import this module. It shares no code with the C++ manager in
libpa and imports nothing from it. Lists, dicts and ``hashlib`` only; every step is
written the plain way (the free queue is a Python list, chain hashes are recomputed
from the start) so that it can be checked against the policy by eye.

Sources (web pages summarising the article "Inside vLLM: Anatomy of a High-Throughput
LLM Inference System"):

* [hn] hn.213312.xyz, "深入解析 vLLM", section 一: the KV-cache manager keeps a queue of
  free blocks (engine construction); allocate_slots works out and allocates the blocks
  a step needs, and the scheduler preempts when they run out (scheduler). Section 二,
  item 2: prefix caching stores a prefix's KV in hashed blocks that later requests
  reuse.
* [blog] shengyayun.com, "读懂 vLLM 推理引擎内幕", section 关键实现细节: item 1, blocks of
  16 tokens, and reuse is block aligned (a partial last block is not reused); item 2,
  each request is hashed per 16-token block (built-in hash by default, SHA-256 against
  collisions), and the longest hit is found by a linear walk over the hash-to-block map.

Readings where the pages are silent (the C++ manager states the same policy):

* B1  The free queue starts as blocks 0..N-1 in id order. Allocation takes its head;
      a block whose last holder lets go joins its tail, a request's last block first.
* B2  Block j's hash is H(hash of block j-1, its 16 token ids as little-endian int32),
      with an all-zero parent for block 0. H is 64-bit FNV-1a over parent(8) ||
      tokens(64), stored as 8 little-endian bytes then 24 zero bytes, or SHA-256 over
      parent(32) || tokens(64).
* B3  A block is hashed (offered to the map) once allocate_slots covers all 16 of its
      tokens and they are known. A hash that already names another block is not
      re-registered.
* B4  A new request's hit is its longest run of leading full blocks whose hashes are
      in the map, at most (n - 1) // 16 blocks so that one token is still computed. The
      hit blocks are claimed at registration and count as computed.
* B5  A cached block keeps its hash while it waits in the free queue; it loses it
      (eviction) when allocation takes it.
"""

from __future__ import annotations

import hashlib

BLOCK = 16


class NoSpace(Exception):
    """Too few free blocks; nothing changed."""


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: start at the offset basis, then per byte xor it in and multiply by
    the FNV prime, modulo 2**64."""
    h = 0xCBF29CE484222325
    for byte in data:
        h ^= byte
        h = (h * 0x100000001B3) % (1 << 64)
    return h


def block_hash(kind: str, parent: bytes, tokens) -> bytes:
    """B2: the hash of one full block given its parent's hash (32 bytes)."""
    assert len(tokens) == BLOCK
    payload = b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    if kind == "sha256":
        return hashlib.sha256(parent[:32] + payload).digest()
    if kind == "fnv1a64":
        return fnv1a64(parent[:8] + payload).to_bytes(8, "little") + bytes(24)
    raise ValueError(kind)


def chain_hashes(kind: str, tokens, num_blocks: int) -> list[bytes]:
    """Hashes of the first ``num_blocks`` full blocks of ``tokens``, parent first."""
    out = []
    parent = bytes(32)
    for j in range(num_blocks):
        parent = block_hash(kind, parent, tokens[BLOCK * j: BLOCK * (j + 1)])
        out.append(parent)
    return out


class BlockManagerModel:
    def __init__(self, num_blocks: int, prefix_caching: bool = True, hash: str = "sha256"):
        assert num_blocks >= 1
        self.num_blocks = num_blocks
        self.prefix_caching = prefix_caching
        self.kind = hash
        self.free = list(range(num_blocks))  # B1: index 0 is the head
        self.ref = [0] * num_blocks
        self.block_key = [None] * num_blocks  # hash a block is registered under
        self.cached = {}  # hash -> block
        self.requests = {}

    # -- requests ----------------------------------------------------------------------

    def add_request(self, rid: int, tokens) -> int:
        if rid in self.requests:
            raise KeyError(f"request {rid} already registered")
        tokens = [int(t) for t in tokens]
        assert len(tokens) >= 1
        hit_blocks = []
        if self.prefix_caching:  # B4
            max_hit = (len(tokens) - 1) // BLOCK
            for h in chain_hashes(self.kind, tokens, max_hit):
                if h not in self.cached:
                    break
                hit_blocks.append(self.cached[h])
        for b in hit_blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        n_hit = len(hit_blocks) * BLOCK
        self.requests[rid] = {"tokens": tokens, "blocks": list(hit_blocks), "computed": n_hit, "hit": n_hit,
                              "registered": len(hit_blocks)}
        return n_hit

    def append_tokens(self, rid: int, tokens) -> None:
        self.requests[rid]["tokens"].extend(int(t) for t in tokens)

    def allocate_slots(self, rid: int, num_new: int) -> None:
        r = self.requests[rid]
        assert num_new >= 1
        upto = r["computed"] + num_new
        if upto > len(r["tokens"]):
            raise ValueError("tokens not known yet")
        want = -(-upto // BLOCK)
        need = want - len(r["blocks"])
        if need > len(self.free):
            raise NoSpace(f"need {need}, {len(self.free)} free")
        for _ in range(max(need, 0)):
            b = self.free.pop(0)
            if self.block_key[b] is not None:  # B5: eviction
                if self.cached.get(self.block_key[b]) == b:
                    del self.cached[self.block_key[b]]
                self.block_key[b] = None
            self.ref[b] = 1
            r["blocks"].append(b)
        if self.prefix_caching:  # B3
            full = upto // BLOCK
            hashes = chain_hashes(self.kind, r["tokens"], full)
            for j in range(r["registered"], full):
                b = r["blocks"][j]
                if self.block_key[b] is None and hashes[j] not in self.cached:
                    self.cached[hashes[j]] = b
                    self.block_key[b] = hashes[j]
            r["registered"] = max(r["registered"], full)

    def free_request(self, rid: int) -> None:
        r = self.requests.pop(rid)
        for b in reversed(r["blocks"]):  # B1
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- one step's arrays ---------------------------------------------------------------

    def build_step(self, rids, query_lens, max_blocks_per_seq: int, num_tokens: int | None = None) -> dict:
        S = len(rids)
        assert len(set(rids)) == S
        for rid, n in zip(rids, query_lens):
            r = self.requests[rid]
            if r["computed"] + n > min(len(r["blocks"]) * BLOCK, len(r["tokens"])):
                raise ValueError(f"request {rid}: query tokens not covered")
            if len(r["blocks"]) > max_blocks_per_seq:
                raise ValueError("block table too narrow")
        T = sum(query_lens) if num_tokens is None else num_tokens
        assert T >= sum(query_lens)
        block_tables = [[0] * max_blocks_per_seq for _ in range(S)]
        ctx, seq_lens, qsl, slots = [], [], [0], []
        for i, (rid, n) in enumerate(zip(rids, query_lens)):
            r = self.requests[rid]
            for j, b in enumerate(r["blocks"]):
                block_tables[i][j] = b
            ctx.append(r["computed"])
            seq_lens.append(r["computed"] + n)
            for pos in range(r["computed"], r["computed"] + n):
                slots.append(r["blocks"][pos // BLOCK] * BLOCK + pos % BLOCK)
            qsl.append(qsl[-1] + n)
            r["computed"] += n
        slots += [-1] * (T - len(slots))
        return {"block_tables": block_tables, "seq_lens": seq_lens, "query_start_loc": qsl, "context_lens": ctx,
                "slot_mapping": slots}

    # -- state, for comparisons ----------------------------------------------------------

    def request_blocks(self, rid: int) -> list[int]:
        return list(self.requests[rid]["blocks"])

    def request_info(self, rid: int) -> dict:
        r = self.requests[rid]
        return {"known_tokens": len(r["tokens"]), "computed_tokens": r["computed"], "cache_hit_tokens": r["hit"],
                "blocks": len(r["blocks"])}

    def block_state(self, b: int) -> tuple[int, int]:
        return self.ref[b], (self.free.index(b) if b in self.free else -1)

    @property
    def num_free_blocks(self) -> int:
        return len(self.free)

    @property
    def num_cached_blocks(self) -> int:
        return len(self.cached)
