"""The seeded generator: shapes, determinism and the structure of each workload."""

import numpy as np
import pytest
import torch

import workload

BS = 16


@pytest.mark.parametrize("name", sorted(workload.CONFIGS))
def test_small_config_structure(name):
    step = workload.make_config(name, small=True)
    ctx, qlen, L = step.lengths()
    assert (L == ctx + qlen).all()
    assert step.query_start_loc[0].item() == 0 and step.query_start_loc[-1].item() == step.num_tokens
    need = (L + BS - 1) // BS
    bt = step.block_tables.numpy()
    assert need.max() <= bt.shape[1]
    for i in range(step.num_seqs):
        row = bt[i, : need[i]]
        assert ((row >= 0) & (row < step.num_blocks)).all()
        assert (bt[i, need[i]:] == -1).all()
    assert step.k_cache.shape == (step.num_blocks, step.num_kv_heads, BS, step.head_dim)
    assert step.v_cache.shape == (step.num_blocks, step.num_kv_heads, step.head_dim, BS)


def test_seeded_and_deterministic():
    a = workload.make_config("mixed_step_bf16", small=True, seed=3)
    b = workload.make_config("mixed_step_bf16", small=True, seed=3)
    c = workload.make_config("mixed_step_bf16", small=True, seed=4)
    for f in ("q", "k", "v", "k_cache", "v_cache", "block_tables", "seq_lens"):
        x, y = getattr(a, f), getattr(b, f)
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), f
    assert not torch.equal(a.q.view(torch.int16), c.q.view(torch.int16))


def test_private_blocks_are_distinct_and_prefix_shared():
    step = workload.make_config("prefix_shared_bf16", small=True)
    ctx, qlen, L = step.lengths()
    bt = step.block_tables.numpy()
    n_shared = 64 // BS
    assert (bt[:, :n_shared] == bt[0, :n_shared]).all()
    private = np.concatenate([bt[i, n_shared: (L[i] + BS - 1) // BS] for i in range(step.num_seqs)])
    assert np.unique(private).size == private.size
    assert not np.isin(private, bt[0, :n_shared]).any()


def test_poison_marks_exactly_the_unfilled_slots():
    step = workload.build_step([5, 16, 0], [1, 3, 2], num_q_heads=2, num_kv_heads=1, head_dim=4,
                               dtype="f32", num_blocks=6, seed=1)
    kc = step.k_cache.numpy()
    bt = step.block_tables.numpy()
    live = np.zeros((6, BS), bool)
    for i, c in enumerate([5, 16, 0]):
        for j in range(c):
            live[bt[i, j // BS], j % BS] = True
    assert (np.isfinite(kc[:, 0, :, 0]) == live).all()
    assert (np.isfinite(step.v_cache.numpy()[:, 0, 0, :]) == live).all()


def test_full_size_lengths_match_the_workload_text():
    # lengths only (no pool) -- reconstruct the draws the builders make
    rng = np.random.default_rng(np.random.SeedSequence([0, 0x1E46]))
    L = rng.integers(512, 4096, size=64, endpoint=True)
    assert L.min() >= 512 and L.max() <= 4096
    rng = np.random.default_rng(np.random.SeedSequence([0, 0x1E46]))
    ctx = rng.integers(1024, 8192, size=1664, endpoint=True)
    assert 1664 + 3 * 2048 == 7808 <= 8192
    assert (ctx + 1 <= 512 * BS).all()


def test_random_slots_distinct_with_padding():
    s = workload.random_slots(100, 10, pad_fraction=0.25, seed=2)
    live = s[s >= 0]
    assert np.unique(live).size == live.size and (live < 160).all() and (s == -1).sum() > 0


def test_mixed_step_table_fits_every_seed():
    """The full-size mixed step's block tables hold the longest sequence any seed can draw
    (a decode row with 8192 cached tokens plus its new one needs 513 blocks)."""
    import inspect

    width = inspect.signature(workload.configs.mixed_step_bf16).parameters["max_blocks_per_seq"].default
    assert width * BS >= 8192 + 1
    for seed in range(64):
        ctx, qlen = workload.configs.mixed_step_lengths(seed)
        assert int(((ctx + qlen + BS - 1) // BS).max()) <= width, seed
        assert int(qlen.sum()) == 7808
