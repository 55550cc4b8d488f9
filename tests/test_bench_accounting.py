"""The algorithmic work bench.py divides by: bytes and flops per step, on the CPU.

Each figure is checked against a count made here another way (a loop over rows, or over
physical blocks) and against the literal value for the full-size workloads.
"""

import numpy as np
import torch

import bench
import workload
from workload.configs import mixed_step_lengths


class _LengthsOnly:
    """What step_work reads of a step, without the pools (the mixed step's are 31 GB)."""

    def __init__(self, ctx, qlen, hq, hkv, d, dtype, width):
        self._ctx, self._qlen = np.asarray(ctx, np.int64), np.asarray(qlen, np.int64)
        self.num_q_heads, self.num_kv_heads, self.head_dim, self.dtype = hq, hkv, d, dtype
        L = self._ctx + self._qlen
        # distinct physical blocks per sequence, as a private pool would deal them out
        bt = np.full((len(L), width), -1, np.int64)
        nxt = 0
        for i, n in enumerate((L + 15) // 16):
            bt[i, :n] = np.arange(nxt, nxt + n)
            nxt += n
        self.block_tables = torch.from_numpy(bt.astype(np.int32))

    def lengths(self):
        return self._ctx, self._qlen, self._ctx + self._qlen


def test_mixed_step_work():
    ctx, qlen = mixed_step_lengths()
    work = bench.step_work(_LengthsOnly(ctx, qlen, 32, 8, 128, "bf16", 513))
    tok = 8 * 128 * 2 * 2  # K and V of one token over 8 kv heads, bf16
    dec = qlen == 1
    assert work["decode_rows"] == work["decode_path_seqs"] == 1664 and work["chunk_seqs"] == 3
    assert work["decode_kv_bytes"] == sum(int(c) + 1 for c in ctx[dec]) * tok == 31_133_310_976
    # private blocks: unique bytes equal the logical ones
    assert work["decode_kv_unique_bytes"] == work["decode_kernel_kv_bytes"] == work["decode_kv_bytes"]
    pairs = sum(int(c) + j + 1 for c, n in zip(ctx[~dec], qlen[~dec]) for j in range(int(n)))
    assert work["prefill_causal_pairs_per_head"] == pairs == 23_071_744
    assert work["prefill_flops"] == 4 * 128 * 32 * pairs == 378_007_453_696
    assert work["attn_f32_flops"] == 0 and work["prefix_flops"] == 0
    assert work["scatter_bytes"] == 7808 * tok * 2


def test_prefix_shared_work():
    """128 decode rows over one 4096-token prefix: logical bytes count it per row, unique
    bytes once, and the decode kernel reads only the suffixes."""
    step = workload.make_config("prefix_shared_bf16")
    ctx, qlen, L = step.lengths()
    work = bench.step_work(step, prefix_keys=4096)
    tok = step.num_kv_heads * step.head_dim * 2 * 2
    assert work["decode_kv_bytes"] == int(L.sum()) * tok == 2_425_622_528
    bt = step.block_tables.numpy()
    fill = {}
    for i in range(step.num_seqs):
        for t in range(int(L[i])):
            fill.setdefault(int(bt[i, t // 16]), set()).add(t % 16)
    assert work["decode_kv_unique_bytes"] == sum(len(v) for v in fill.values()) * tok == 294_916_096
    assert work["decode_kernel_kv_bytes"] == (int(L.sum()) - 128 * 4096) * tok
    assert work["prefix_flops"] == 4 * step.head_dim * step.num_q_heads * 128 * 4096


def test_spec_verify_work():
    """Multi-row sequences of 4 rows (G = 4) take the decode path: their keys count as
    decode bytes, and there are no decode rows of one token."""
    ctx = [500, 1000]
    work = bench.step_work(_LengthsOnly(ctx, [4, 4], 32, 8, 128, "bf16", 128))
    assert work["decode_path_seqs"] == 2 and work["decode_rows"] == 0 and work["chunk_seqs"] == 0
    assert work["decode_kv_bytes"] == (504 + 1004) * 8 * 128 * 4
    assert work["prefill_flops"] == 0


def test_f32_work():
    """An fp32 step: one kernel attends every row, so its flops cover all causal pairs."""
    ctx, qlen = [0, 3, 17], [1, 5, 2]
    work = bench.step_work(_LengthsOnly(ctx, qlen, 4, 1, 64, "f32", 4))
    pairs = sum(c + j + 1 for c, n in zip(ctx, qlen) for j in range(n))
    assert work["attn_f32_flops"] == 4 * 64 * 4 * pairs
