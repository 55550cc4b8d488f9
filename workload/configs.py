"""The five synthetic step workloads, plus reduced-size variants for quick tests.

Each workload follows the structure the pages give for a serving step: KV in
16-token blocks; a step that mixes decode tokens with chunks of long prompts under a
token budget; requests whose block lists share a prefix; and long contexts.  The
pages print no workload data (their own measurements use a model and a chat dataset
that are not available), so these seeded draws stand in for them.

Lengths are integer draws, uniform and inclusive.  A sequence's ``seq_len`` counts
the token(s) of this step: ``seq_len = context_len + query_len``.
"""

from __future__ import annotations

import numpy as np

from .step import BLOCK_SIZE, Step, build_step


def _lengths_rng(seed: int):
    return np.random.default_rng(np.random.SeedSequence([seed, 0x1E46]))


def tiny_decode_f32(seed: int = 0, device="cpu", **kw) -> Step:
    """4 decode sequences of 1/17/33/50 tokens, fp32, 4 q heads over 1 kv head, D=64, 32-block pool."""
    L = np.array([1, 17, 33, 50])
    return build_step(L - 1, np.ones(4, np.int64), num_q_heads=4, num_kv_heads=1, head_dim=64,
                      dtype="f32", scale=1.0 / 8.0, num_blocks=32, max_blocks_per_seq=4,
                      seed=seed, device=device, name="tiny_decode_f32", **kw)


def decode_batch_bf16(seed: int = 0, device="cpu", num_seqs: int = 64, lo: int = 512, hi: int = 4096,
                      num_blocks: int = 20000, max_blocks_per_seq: int = 256, **kw) -> Step:
    """64 decode sequences, seq_len ~ U[512, 4096], 32/8 heads, D=128, pool of 20000 blocks."""
    L = _lengths_rng(seed).integers(lo, hi, size=num_seqs, endpoint=True)
    return build_step(L - 1, np.ones(num_seqs, np.int64), num_q_heads=32, num_kv_heads=8, head_dim=128,
                      dtype="bf16", num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq,
                      seed=seed, device=device, name="decode_batch_bf16", **kw)


def mixed_step_lengths(seed: int = 0, num_decode: int = 1664, ctx_lo: int = 1024, ctx_hi: int = 8192,
                       chunk: int = 2048, chunk_ctx=(0, 2048, 6144)):
    """(context_lens, query_lens) of the mixed step: decode rows first, then the chunks."""
    ctx_dec = _lengths_rng(seed).integers(ctx_lo, ctx_hi, size=num_decode, endpoint=True)
    ctx = np.concatenate([ctx_dec, np.asarray(chunk_ctx, np.int64)])
    qlen = np.concatenate([np.ones(num_decode, np.int64), np.full(len(chunk_ctx), chunk, np.int64)])
    return ctx, qlen


def mixed_step_bf16(seed: int = 0, device="cpu", num_decode: int = 1664, ctx_lo: int = 1024,
                    ctx_hi: int = 8192, chunk: int = 2048, chunk_ctx=(0, 2048, 6144),
                    max_blocks_per_seq: int = 513, **kw) -> Step:
    """1664 decode tokens (context ~ U[1024, 8192]) then three 2048-token prefill chunks whose
    cached context is 0, 2048 and 6144 tokens: 7808 tokens under an 8192-token budget. The
    block tables are 513 blocks wide, room for a decode row with 8192 cached tokens plus
    its new one."""
    ctx, qlen = mixed_step_lengths(seed, num_decode, ctx_lo, ctx_hi, chunk, chunk_ctx)
    return build_step(ctx, qlen, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                      max_blocks_per_seq=max_blocks_per_seq, seed=seed, device=device,
                      name="mixed_step_bf16", **kw)


def prefix_shared_bf16(seed: int = 0, device="cpu", num_seqs: int = 128, prefix: int = 4096,
                       lo: int = 64, hi: int = 1024, max_blocks_per_seq: int = 320, **kw) -> Step:
    """128 decode sequences listing the same 256 blocks (a 4096-token prefix) first, then
    private suffixes of U[64, 1024] tokens (the new token included); 64/8 heads, D=128."""
    suffix = _lengths_rng(seed).integers(lo, hi, size=num_seqs, endpoint=True)
    L = prefix + suffix
    return build_step(L - 1, np.ones(num_seqs, np.int64), num_q_heads=64, num_kv_heads=8, head_dim=128,
                      dtype="bf16", shared_prefix_tokens=prefix, max_blocks_per_seq=max_blocks_per_seq,
                      seed=seed, device=device, name="prefix_shared_bf16", **kw)


def long_decode_bf16(seed: int = 0, device="cpu", num_seqs: int = 16, seq_len: int = 131072, **kw) -> Step:
    """16 decode sequences of 131072 tokens (8192 blocks each), 64/8 heads, D=128, shuffled pool."""
    L = np.full(num_seqs, seq_len, np.int64)
    nb = num_seqs * ((seq_len + BLOCK_SIZE - 1) // BLOCK_SIZE)
    return build_step(L - 1, np.ones(num_seqs, np.int64), num_q_heads=64, num_kv_heads=8, head_dim=128,
                      dtype="bf16", num_blocks=nb, max_blocks_per_seq=(seq_len + BLOCK_SIZE - 1) // BLOCK_SIZE,
                      seed=seed, device=device, name="long_decode_bf16", **kw)


def spec_verify_bf16(seed: int = 0, device="cpu", num_seqs: int = 64, rows: int = 4, lo: int = 512, hi: int = 4096,
                     max_blocks_per_seq: int = 256, **kw) -> Step:
    """Speculative-decoding verification step: 64 sequences each verifying 3 drafted tokens
    (4 query rows: the drafts plus the last accepted token), context ~ U[512, 4096];
    32/8 heads, D=128. The pages' example drafts 3 tokens per step."""
    ctx = _lengths_rng(seed).integers(lo, hi, size=num_seqs, endpoint=True)
    return build_step(ctx, np.full(num_seqs, rows, np.int64), num_q_heads=32, num_kv_heads=8, head_dim=128,
                      dtype="bf16", max_blocks_per_seq=max_blocks_per_seq, seed=seed, device=device,
                      name="spec_verify_bf16", **kw)


CONFIGS = {
    "tiny_decode_f32": tiny_decode_f32,
    "decode_batch_bf16": decode_batch_bf16,
    "mixed_step_bf16": mixed_step_bf16,
    "prefix_shared_bf16": prefix_shared_bf16,
    "long_decode_bf16": long_decode_bf16,
    "spec_verify_bf16": spec_verify_bf16,
}

# Reduced sizes with the same structure; the oracle finishes these in seconds.
SMALL = {
    "tiny_decode_f32": {},
    "decode_batch_bf16": dict(num_seqs=6, lo=20, hi=300, num_blocks=200, max_blocks_per_seq=24),
    "mixed_step_bf16": dict(num_decode=5, ctx_lo=10, ctx_hi=300, chunk=70, chunk_ctx=(0, 33, 100),
                            max_blocks_per_seq=24),
    "prefix_shared_bf16": dict(num_seqs=5, prefix=64, lo=1, hi=40, max_blocks_per_seq=8),
    "long_decode_bf16": dict(num_seqs=2, seq_len=1500),
    "spec_verify_bf16": dict(num_seqs=5, lo=0, hi=200, max_blocks_per_seq=16),
}


def make_config(name: str, *, small: bool = False, seed: int = 0, device="cpu", **kw) -> Step:
    """Build workload ``name`` (full size, or the reduced variant with ``small=True``)."""
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    args = dict(SMALL[name]) if small else {}
    args.update(kw)
    return CONFIGS[name](seed=seed, device=device, **args)
