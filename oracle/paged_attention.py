"""Plain fp64 CPU definition of one paged-attention step -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import or run this module.  It shares no code, header, table or helper with the HIP
library and imports nothing from it; it is slow on purpose and written so that each
step can be checked against the text it follows by eye.

Sources (three web pages summarising the article "Inside vLLM: Anatomy of a
High-Throughput LLM Inference System"):

* [news]  chat-gpts.plus news summary, section "事件核心" (what happened);
* [hn]    hn.213312.xyz restatement "深入解析 vLLM：高性能 LLM 推理系统剖析",
          section 一 (engine and engine core: scheduler, forward pass) and 二 (chunked
          prefill, prefix caching);
* [blog]  shengyayun.com "读懂 vLLM 推理引擎内幕", section "关键实现细节" items ① (memory
          ledger: 16-token blocks) and ② (prefix caching by 16-token blocks).

What the pages fix, restated:

* KV is stored in fixed-size blocks that are handed out and taken back as needed
  ([news] 事件核心; [blog] 关键实现细节 ①, default block = 16 tokens).
* Before each forward pass the worker prepares, among its inputs, the positions of the
  step's tokens and the slot mapping (where each token's K/V go); every scheduled
  sequence is flattened into one concatenated "super-sequence" and a custom
  paged-attention kernel runs over it ([hn] §一, forward pass).
* A step mixes decode requests with prefill; long prompts are cut into chunks that run
  over several steps ([hn] §一 scheduler, §二 item 1).
* Requests may list the same KV blocks (prefix reuse, whole 16-token blocks only)
  ([blog] 关键实现细节 ②; [hn] §二 item 2).

Where the pages are silent, this oracle takes the following readings:

* R1  Pool layout: ``k_cache[b, h, o, d]`` and ``v_cache[b, h, d, o]`` hold dimension d of
      kv head h of the token in slot ``16*b + o`` (keys token-major, values dim-major
      inside each block).
* R2  A slot is ``block_id * 16 + offset``.
* R3  Row r of sequence i is the token at position ``context_lens[i] + r``.
* R4  Causal mask: the token at position p sees keys 0..p of its own sequence (all of
      its cached context, and its chunk up to itself).
* R5  Query head h reads kv head ``h // (Hq // Hkv)`` (contiguous groups).
* R6  ``seq_lens[i] = context_lens[i] + query_len[i]``; all three are checked.
* R8  A negative slot means "do not write this token".
* R9  Non-negative slots must be distinct (otherwise the write has no single result).
* R10 The softmax scale is an argument.
* R15 Sequences with no query rows produce no output rows.

Attention itself is ordinary softmax attention of each row over the keys it sees,
taken in logical order: paging only decides where the numbers are stored, so it is
the same sum as contiguous causal attention.
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16  # tokens per KV block ([blog] 关键实现细节 ①)


class OracleInputError(ValueError):
    """The inputs break a precondition of the step (see ``validate_step``)."""


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 copy of a payload array.

    ``float32`` arrays widen directly; ``uint16`` arrays hold bfloat16 bit patterns,
    which are the upper 16 bits of a float32 and widen exactly the same way.
    """
    if x.dtype == np.float32:
        return x.astype(np.float64)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float64:
        return x.copy()
    raise TypeError(f"unsupported payload dtype {x.dtype}")


def slot_mapping(block_tables, query_start_loc, context_lens):
    """Positions and cache slots of the step's tokens ([hn] §一 forward-pass inputs).

    Token t = query_start_loc[i] + r of sequence i sits at position
    p = context_lens[i] + r (R3); its slot is block_tables[i][p // 16] * 16 + p % 16 (R2).
    Returns ``(positions int32 [T], slots int64 [T])``.
    """
    bt = np.asarray(block_tables)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    num_tokens = int(qsl[-1]) if qsl.size else 0
    positions = np.zeros(num_tokens, dtype=np.int32)
    slots = np.zeros(num_tokens, dtype=np.int64)
    for i in range(ctx.shape[0]):
        for t in range(int(qsl[i]), int(qsl[i + 1])):
            p = int(ctx[i]) + (t - int(qsl[i]))
            positions[t] = p
            slots[t] = int(bt[i, p // BLOCK_SIZE]) * BLOCK_SIZE + p % BLOCK_SIZE
    return positions, slots


def reshape_and_cache(k, v, k_cache, v_cache, slots):
    """Write each token's K and V into its slot; returns new pools (inputs untouched).

    For every token t with s = slots[t] >= 0 (R8):
    ``K[s // 16, :, s % 16, :] = k[t]`` and ``V[s // 16, :, :, s % 16] = v[t]`` (R1, R2).
    A pure copy: the stored bits are the input bits.
    """
    new_k = k_cache.copy()
    new_v = v_cache.copy()
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        b, o = divmod(int(s), BLOCK_SIZE)
        new_k[b, :, o, :] = k[t]
        new_v[b, :, :, o] = v[t]
    return new_k, new_v


def gather_sequence(k_cache, v_cache, table_row, length):
    """Keys and values of one sequence in logical order, widened to fp64.

    Logical token j lives in block ``table_row[j // 16]`` at offset ``j % 16``.
    Returns ``K, V`` of shape ``[length, Hkv, D]``.
    """
    n_blocks = (int(length) + BLOCK_SIZE - 1) // BLOCK_SIZE
    ids = np.asarray(table_row[:n_blocks], dtype=np.int64)
    kb = k_cache[ids]                               # [nb, Hkv, 16, D]
    vb = v_cache[ids]                               # [nb, Hkv, D, 16]
    keys = kb.transpose(0, 2, 1, 3)                 # [nb, 16, Hkv, D]
    vals = vb.transpose(0, 3, 1, 2)                 # [nb, 16, Hkv, D]
    hkv, d = keys.shape[2], keys.shape[3]
    keys = keys.reshape(n_blocks * BLOCK_SIZE, hkv, d)[:length]
    vals = vals.reshape(n_blocks * BLOCK_SIZE, hkv, d)[:length]
    return widen(np.ascontiguousarray(keys)), widen(np.ascontiguousarray(vals))


def validate_step(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens,
                  slots=None):
    """Raise ``OracleInputError`` if the step breaks a precondition (R2, R6, R9)."""
    bt = np.asarray(block_tables)
    L = np.asarray(seq_lens, dtype=np.int64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = ctx.shape[0]
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.ndim != 4:
        raise OracleInputError("q must be [T, Hq, D]; pools must be 4-D")
    T, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    if k_cache.shape != (nb, hkv, BLOCK_SIZE, d) or v_cache.shape != (nb, hkv, d, BLOCK_SIZE):
        raise OracleInputError("pool shapes must be [NB, Hkv, 16, D] (keys) and [NB, Hkv, D, 16] (values)")
    if hkv == 0 or hq % hkv:
        raise OracleInputError("Hq must be a positive multiple of Hkv")
    if L.shape != (S,) or qsl.shape != (S + 1,) or bt.ndim != 2 or bt.shape[0] != S:
        raise OracleInputError("length arrays / block table have inconsistent sizes")
    if S and (qsl[0] != 0 or (np.diff(qsl) < 0).any() or qsl[-1] != T):
        raise OracleInputError("query_start_loc must start at 0, not decrease and end at T")
    if (ctx < 0).any() or (L != ctx + np.diff(qsl)).any():
        raise OracleInputError("seq_lens must equal context_lens + query length")
    need = (L + BLOCK_SIZE - 1) // BLOCK_SIZE
    if S and need.max() > bt.shape[1]:
        raise OracleInputError("a sequence needs more blocks than its block-table row holds")
    for i in range(S):
        row = bt[i, : need[i]]
        if ((row < 0) | (row >= nb)).any():
            raise OracleInputError(f"sequence {i} lists a block id outside [0, {nb})")
    if slots is not None:
        s = np.asarray(slots, dtype=np.int64)
        if ((s < -1) | (s >= nb * BLOCK_SIZE)).any():
            raise OracleInputError("slot outside [-1, 16*NB)")
        live = s[s >= 0]
        if np.unique(live).size != live.size:
            raise OracleInputError("two tokens share a slot")


def attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale,
              rows=None, require_finite=True):
    """Softmax attention of every query row over the keys it sees, in fp64.

    The pools passed in must already hold this step's tokens (``reshape_and_cache``
    runs first; the attention call reads the new tokens back from the cache).

    For row t = query_start_loc[i] + r of sequence i, at position p = context_lens[i] + r,
    and query head h with kv head g = h // G (R5):
        s_j   = scale * sum_d q[t, h, d] * K_i[j, g, d]     for j = 0..p   (R4)
        out   = sum_j exp(s_j - max s) * V_i[j, g, :]  /  sum_j exp(s_j - max s)
    ``rows`` (optional) limits the work to those token indices; other rows are NaN.
    Returns ``[T, Hq, D]`` float64, unrounded.
    """
    bt = np.asarray(block_tables)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    T, hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    out = np.full((T, hq, d), np.nan, dtype=np.float64)
    wanted = None
    if rows is not None:
        wanted = np.zeros(T, dtype=bool)
        wanted[np.asarray(rows, dtype=np.int64)] = True
    for i in range(ctx.shape[0]):
        t0, t1 = int(qsl[i]), int(qsl[i + 1])
        r_sel = np.arange(t1 - t0)
        if wanted is not None:
            r_sel = r_sel[wanted[t0:t1]]
        if r_sel.size == 0:
            continue
        pos = ctx[i] + r_sel                               # positions of the chosen rows
        last = int(pos.max())                              # furthest key any chosen row sees
        keys, vals = gather_sequence(k_cache, v_cache, bt[i], int(L[i]))
        keys, vals = keys[: last + 1], vals[: last + 1]
        if require_finite and not (np.isfinite(keys).all() and np.isfinite(vals).all()):
            raise OracleInputError(f"sequence {i} reads a slot that holds no finite token")
        visible = np.arange(last + 1)[None, :] <= pos[:, None]         # [rows, keys]
        qrows = widen(np.ascontiguousarray(q[t0 + r_sel]))             # [rows, Hq, D]
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)
            qg = qrows[:, heads, :].reshape(-1, d)                      # [rows*G, D]
            scores = scale * (qg @ keys[:, g, :].T)                     # [rows*G, keys]
            mask = np.repeat(visible, group, axis=0)
            scores = np.where(mask, scores, -np.inf)
            peak = scores.max(axis=1, keepdims=True)
            weights = np.where(mask, np.exp(scores - peak), 0.0)
            o = (weights @ vals[:, g, :]) / weights.sum(axis=1, keepdims=True)
            out[t0 + r_sel, heads, :] = o.reshape(r_sel.size, group, d)
    return out
