"""PA_DEBUG=1: index checks that run before any work is enqueued.

Every broken input here is built so that even an unchecked run would stay inside its
allocations (the block table has a padding row on each side, and the pools have a
spare block past num_blocks). The checks must refuse each one with PA_E_INDEX and
name the first violation. A valid step must give the same bits with and without
the checks.
"""

import numpy as np
import pytest
import torch

import workload
from gpu_support import gpu_step, log, require_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"
PA_E_INDEX = 10


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("PA_DEBUG", "1")


def _bits(t):
    return t.view(torch.int16)


def _padded(step):
    """The step's block table inside a larger one (one padding row on each side), and
    pools with one spare block past num_blocks; returns views with the step's shapes."""
    S, MB = step.block_tables.shape
    big = torch.zeros(S + 2, MB, dtype=torch.int32, device=DEV)
    big[1:S + 1] = step.block_tables
    nb = step.k_cache.shape[0]
    kc = torch.zeros((nb + 1,) + tuple(step.k_cache.shape[1:]), dtype=step.k_cache.dtype, device=DEV)
    vc = torch.zeros((nb + 1,) + tuple(step.v_cache.shape[1:]), dtype=step.v_cache.dtype, device=DEV)
    kc[:nb] = step.k_cache
    vc[:nb] = step.v_cache
    return big, big[1:S + 1], kc, vc, kc[:nb], vc[:nb]


def _step():
    return workload.build_step([20, 0, 40, 7], [1, 30, 1, 5], num_q_heads=8, num_kv_heads=2, head_dim=128,
                               dtype="bf16", num_blocks=24, max_blocks_per_seq=6, seed=12, device=DEV)


def test_debug_mode_valid_step_is_unchanged(monkeypatch):
    import paged_kv_cache_460_amd as pa

    step = _step()
    monkeypatch.setenv("PA_DEBUG", "0")
    ref = gpu_step(step)  # checks off
    monkeypatch.setenv("PA_DEBUG", "1")
    kc, vc = step.k_cache.clone(), step.v_cache.clone()
    out = pa.step(step.q, step.k, step.v, kc, vc, step.block_tables, step.seq_lens, step.query_start_loc,
                  step.context_lens, step.scale)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref["out"]))
    assert torch.equal(_bits(kc), _bits(ref["k_cache"]))


def _expect_index_error(fn, text):
    import paged_kv_cache_460_amd as pa

    with pytest.raises(pa.PAError) as ei:
        fn()
    torch.cuda.synchronize()
    assert ei.value.status == PA_E_INDEX, ei.value
    assert text in str(ei.value), str(ei.value)
    log(f"[debug] refused as expected: {ei.value}")


def _attention(pa, step, bt, kc, vc, seq_lens=None, qsl=None, ctx=None):
    return pa.attention(step.q, kc, vc, bt, step.seq_lens if seq_lens is None else seq_lens,
                        step.query_start_loc if qsl is None else qsl,
                        step.context_lens if ctx is None else ctx, step.scale)


def test_debug_refuses_inconsistent_seq_lens(debug):
    import paged_kv_cache_460_amd as pa

    step = _step()
    _, bt, _, _, kc, vc = _padded(step)
    sl = step.seq_lens.clone()
    sl[2] += 1
    _expect_index_error(lambda: _attention(pa, step, bt, kc, vc, seq_lens=sl), "sequence 2: seq_lens differs")


def test_debug_refuses_block_id_past_the_pool(debug):
    import paged_kv_cache_460_amd as pa

    step = _step()
    _, bt, _, _, kc, vc = _padded(step)
    bt[1, 1] = kc.shape[0]  # the spare block: real memory, but not part of the pool
    _expect_index_error(lambda: _attention(pa, step, bt, kc, vc), "sequence 1: a block id lies outside")


def test_debug_refuses_negative_block_id_in_slot_mapping(debug):
    import paged_kv_cache_460_amd as pa

    step = _step()
    _, bt, _, _, _, _ = _padded(step)
    bt[3, 0] = -1
    _expect_index_error(lambda: pa.build_slot_mapping(bt, step.query_start_loc, step.context_lens,
                                                      num_tokens=step.num_tokens), "sequence 3: a block id")


def test_debug_refuses_decreasing_query_offsets(debug):
    import paged_kv_cache_460_amd as pa

    step = _step()
    _, bt, _, _, kc, vc = _padded(step)
    qsl = step.query_start_loc.clone()
    qsl[2] = qsl[1] - 1  # sequence 1 now has a negative row count
    _expect_index_error(lambda: pa.build_slot_mapping(bt, qsl, step.context_lens, num_tokens=step.num_tokens),
                        "sequence 1: query_start_loc decreases")
    _expect_index_error(lambda: _attention(pa, step, bt, kc, vc, qsl=qsl), "sequence 1: query_start_loc decreases")


def test_debug_refuses_a_sequence_wider_than_its_table(debug):
    import paged_kv_cache_460_amd as pa

    step = _step()
    _, bt, _, _, kc, vc = _padded(step)
    ctx = step.context_lens.clone()
    sl = step.seq_lens.clone()
    ctx[0] += 80  # 101 tokens: 7 blocks in a 6-wide table
    sl[0] += 80
    _expect_index_error(lambda: _attention(pa, step, bt, kc, vc, seq_lens=sl, ctx=ctx),
                        "sequence 0: the sequence needs more than max_blocks_per_seq")


def test_debug_refuses_bad_slots(debug):
    import paged_kv_cache_460_amd as pa

    step = _step()
    _, _, _, _, kc, vc = _padded(step)
    T = step.num_tokens
    good = np.arange(T, dtype=np.int64) + 3
    dup = good.copy()
    dup[T - 2] = dup[5]
    _expect_index_error(lambda: pa.reshape_and_cache(step.k, step.v, kc, vc, torch.from_numpy(dup).to(DEV)),
                        f"token {T - 2}: the slot repeats")
    far = good.copy()
    far[7] = kc.shape[0] * 16  # the spare block's first slot
    _expect_index_error(lambda: pa.reshape_and_cache(step.k, step.v, kc, vc, torch.from_numpy(far).to(DEV)),
                        "token 7: the slot lies outside")
    pa.reshape_and_cache(step.k, step.v, kc, vc, torch.from_numpy(good).to(DEV))  # accepted
    torch.cuda.synchronize()
