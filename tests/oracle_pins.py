"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each ``pin_*`` function takes an oracle module (the real one, or a deliberately broken
copy in the mutation tests) and raises ``AssertionError`` when the module disagrees
with what the definition or mathematics fixes:

* brute force: pure-Python loops over contiguous (unpaged) keys and values;
* a library routine: torch's scaled_dot_product_attention in float64;
* closed forms: single-token sequences, constant keys, per-head constant values,
  a query aligned with one key, a hand-worked slot-mapping example;
* invariants that paging implies: block placement, prefix sharing, sequence order,
  batch composition, chunk boundaries;
* the cache write as a plain copy (every other slot keeps its bits).

The layout restated here independently of the oracle: key ``d`` of kv head ``h`` of
the token in slot ``16*b + o`` sits at ``k_cache[b, h, o, d]``; its value at
``v_cache[b, h, d, o]``.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BS = 16


# ---------------------------------------------------------------------------
# helpers (independent of the oracle)
# ---------------------------------------------------------------------------

def _bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    view = {np.dtype(np.float32): np.uint32, np.dtype(np.uint16): np.uint16, np.dtype(np.float64): np.uint64}[a.dtype]
    return bool(np.array_equal(a.view(view), b.view(view)))


def run_oracle(orc, arrays: dict):
    """slot mapping -> cache write -> attention, all through the module under test."""
    pos, slots = orc.slot_mapping(arrays["block_tables"], arrays["query_start_loc"], arrays["context_lens"])
    kc, vc = orc.reshape_and_cache(arrays["k"], arrays["v"], arrays["k_cache"], arrays["v_cache"], slots)
    out = orc.attention(arrays["q"], kc, vc, arrays["block_tables"], arrays["seq_lens"],
                        arrays["query_start_loc"], arrays["context_lens"], arrays["scale"])
    return pos, slots, kc, vc, out


def _tiny_instance(seed: int):
    """A random tiny paged step built from contiguous per-sequence keys/values.

    Returns (arrays for the oracle, contiguous data for brute force).
    """
    rng = np.random.default_rng(seed)
    hkv, group = [(1, 1), (1, 2), (1, 4), (2, 1), (2, 2)][rng.integers(5)]
    hq = hkv * group
    d = int(rng.choice([2, 4, 8]))
    S = int(rng.integers(1, 5))
    ctx, qlen = [], []
    for _ in range(S):
        n = int(rng.integers(0, 11))
        c = int(rng.integers(0, 41 - n))
        ctx.append(c)
        qlen.append(n)
    L = [c + n for c, n in zip(ctx, qlen)]
    nblk = [(x + BS - 1) // BS for x in L]
    mb = max(max(nblk), 1)
    nb = sum(nblk) + int(rng.integers(0, 4)) + 1
    ids = rng.permutation(nb)
    tables = np.full((S, mb), -1, dtype=np.int64)
    cur = 0
    for i in range(S):
        tables[i, : nblk[i]] = ids[cur: cur + nblk[i]]
        cur += nblk[i]
    keys = [rng.standard_normal((L[i], hkv, d)).astype(np.float32) for i in range(S)]
    vals = [rng.standard_normal((L[i], hkv, d)).astype(np.float32) for i in range(S)]
    q = rng.standard_normal((sum(qlen), hq, d)).astype(np.float32)
    kc = np.full((nb, hkv, BS, d), np.nan, dtype=np.float32)
    vc = np.full((nb, hkv, d, BS), np.nan, dtype=np.float32)
    full_kc, full_vc = kc.copy(), vc.copy()
    for i in range(S):
        for j in range(L[i]):
            b, o = int(tables[i, j // BS]), j % BS
            for g in range(hkv):
                for dd in range(d):
                    full_kc[b, g, o, dd] = keys[i][j, g, dd]
                    full_vc[b, g, dd, o] = vals[i][j, g, dd]
                    if j < ctx[i]:
                        kc[b, g, o, dd] = keys[i][j, g, dd]
                        vc[b, g, dd, o] = vals[i][j, g, dd]
    k_new = np.concatenate([keys[i][ctx[i]:] for i in range(S)]).reshape(-1, hkv, d)
    v_new = np.concatenate([vals[i][ctx[i]:] for i in range(S)]).reshape(-1, hkv, d)
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int64)
    arrays = dict(q=q, k=k_new, v=v_new, k_cache=kc, v_cache=vc, block_tables=tables,
                  seq_lens=np.asarray(L, np.int64), query_start_loc=qsl,
                  context_lens=np.asarray(ctx, np.int64), scale=float(rng.uniform(0.2, 1.5)))
    contiguous = dict(keys=keys, vals=vals, ctx=ctx, qlen=qlen, tables=tables, group=group,
                      full_kc=full_kc, full_vc=full_vc)
    return arrays, contiguous


def _brute_force(arrays, cont):
    """Pure-Python causal softmax attention over contiguous keys/values."""
    q, scale, group = arrays["q"], arrays["scale"], cont["group"]
    T, hq, d = q.shape
    out = np.zeros((T, hq, d))
    t = 0
    for i, (c, n) in enumerate(zip(cont["ctx"], cont["qlen"])):
        K, V = cont["keys"][i], cont["vals"][i]
        for r in range(n):
            p = c + r
            for h in range(hq):
                g = h // group
                s = []
                for j in range(p + 1):
                    acc = 0.0
                    for dd in range(d):
                        acc += float(q[t, h, dd]) * float(K[j, g, dd])
                    s.append(scale * acc)
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = sum(w)
                for dd in range(d):
                    out[t, h, dd] = sum(w[j] * float(V[j, g, dd]) for j in range(p + 1)) / tot
            t += 1
    return out


def _step_arrays(name: str, seed: int = 0, **kw):
    step = workload.make_config(name, small=True, seed=seed, **kw)
    return step, workload.host_arrays(step)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_bruteforce(orc, seeds=range(12)):
    """P1: paged oracle == brute-force contiguous attention (and the cache it writes)."""
    for seed in seeds:
        arrays, cont = _tiny_instance(seed)
        pos, slots, kc, vc, out = run_oracle(orc, arrays)
        assert _bits_equal(kc, cont["full_kc"]) and _bits_equal(vc, cont["full_vc"]), f"seed {seed}: cache"
        ref = _brute_force(arrays, cont)
        if ref.size:
            err = np.max(np.abs(out - ref))
            assert err <= 1e-12, f"seed {seed}: max abs err {err}"


def pin_sdpa(orc, seeds=range(6)):
    """P2: one sequence equals torch SDPA (float64, explicit causal mask with context, GQA)."""
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4]))
        hq, d = hkv * group, int(rng.choice([8, 16, 32]))
        ctx = 0 if seed % 2 == 0 else int(rng.integers(1, 60))
        n = int(rng.integers(1, 40))
        L = ctx + n
        step = workload.build_step([ctx], [n], num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype="f32",
                                   scale=float(rng.uniform(0.1, 1.0)), seed=seed, num_blocks=(L + 15) // 16 + 3)
        arrays = workload.host_arrays(step)
        _, _, kc, vc, out = run_oracle(orc, arrays)
        # contiguous keys/values recovered from the cache through the documented layout
        tbl = arrays["block_tables"][0]
        K = np.stack([kc[tbl[j // BS], :, j % BS, :] for j in range(L)]).astype(np.float64)
        V = np.stack([vc[tbl[j // BS], :, :, j % BS] for j in range(L)]).astype(np.float64)
        qt = torch.from_numpy(arrays["q"].astype(np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(K).permute(1, 0, 2)[None]
        vt = torch.from_numpy(V).permute(1, 0, 2)[None]
        if ctx == 0:
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, is_causal=True, scale=arrays["scale"], enable_gqa=True)
        else:
            mask = torch.arange(L)[None, :] <= (ctx + torch.arange(n))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=mask, scale=arrays["scale"], enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        err = np.max(np.abs(out - ref))
        assert err <= 1e-12, f"seed {seed}: SDPA max abs err {err}"


def pin_single_token(orc):
    """P3(i): a sequence of one token attends only to itself: out == its value, exactly."""
    step, arrays = _step_arrays("tiny_decode_f32")
    _, _, _, _, out = run_oracle(orc, arrays)
    group = arrays["q"].shape[1] // arrays["k"].shape[1]
    expect = np.repeat(arrays["v"][0].astype(np.float64), group, axis=0)
    assert np.array_equal(out[0], expect), "length-1 sequence must return its own value"
    # the same in bfloat16 payloads (checks the exact widening of bf16 bits)
    bstep = workload.build_step([0, 5], [1, 1], num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="bf16", seed=3)
    barr = workload.host_arrays(bstep)
    _, _, _, _, bout = run_oracle(orc, barr)
    vf = bstep.v[0].float().numpy().astype(np.float64)
    assert np.array_equal(bout[0], np.repeat(vf, 2, axis=0)), "bf16 length-1 sequence"


def pin_constant_keys(orc):
    """P3(ii): all keys zero -> uniform weights -> output = mean of values over positions 0..p."""
    ctx, qlen = [0, 21, 40], [19, 1, 7]
    step = workload.build_step(ctx, qlen, num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="f32",
                               seed=5, num_blocks=20)
    arrays = workload.host_arrays(step)
    arrays["k"][:] = 0.0
    kc = arrays["k_cache"]
    kc[np.isfinite(kc)] = 0.0
    # value of logical token j, kv head g, dim d: j*(d+1) + 100*g  (written through the layout)
    L = arrays["seq_lens"]
    vc = arrays["v_cache"]
    qsl = arrays["query_start_loc"]
    for i in range(3):
        for j in range(int(L[i])):
            for g in range(2):
                val = (j * (np.arange(8) + 1) + 100 * g).astype(np.float32)
                if j < ctx[i]:
                    vc[arrays["block_tables"][i, j // BS], g, :, j % BS] = val
                else:
                    arrays["v"][qsl[i] + j - ctx[i], g, :] = val
    _, _, _, _, out = run_oracle(orc, arrays)
    for i in range(3):
        for r in range(qlen[i]):
            p = ctx[i] + r
            for h in range(4):
                expect = (p / 2.0) * (np.arange(8) + 1) + 100 * (h // 2)
                err = np.max(np.abs(out[qsl[i] + r, h] - expect))
                assert err <= 1e-10, f"seq {i} row {r} head {h}: {err}"


def pin_group_mapping(orc):
    """P3(iii): values of kv head g are all g -> query head h returns h // G."""
    def bf16_bits(x: float) -> np.uint16:
        return torch.tensor([x], dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]

    def is_nan_bits(x: np.ndarray) -> np.ndarray:
        return ((x & 0x7F80) == 0x7F80) & ((x & 0x007F) != 0)

    for hq, hkv in [(8, 2), (6, 3), (16, 4), (4, 1)]:
        step = workload.build_step([10, 30], [3, 1], num_q_heads=hq, num_kv_heads=hkv, head_dim=4,
                                   dtype="bf16", seed=7)
        arrays = workload.host_arrays(step)
        vc, vn = arrays["v_cache"].copy(), arrays["v"].copy()
        for g in range(hkv):
            head = vc[:, g]
            head[~is_nan_bits(head)] = bf16_bits(float(g))   # poisoned slots stay poisoned
            vn[:, g] = bf16_bits(float(g))
        arrays["v_cache"], arrays["v"] = vc, vn
        _, _, _, _, out = run_oracle(orc, arrays)
        group = hq // hkv
        for h in range(hq):
            err = np.max(np.abs(out[:, h, :] - h // group))
            assert err <= 1e-12, f"Hq={hq} Hkv={hkv}: head {h}: {err}"


def pin_aligned_query(orc):
    """P3(iv): a query that is a large multiple of one key picks out that key's value."""
    step = workload.build_step([37, 0], [1, 18], num_q_heads=2, num_kv_heads=1, head_dim=16, dtype="f32",
                               seed=11, num_blocks=9)
    arrays = workload.host_arrays(step)
    tbl = arrays["block_tables"]
    for target in (0, 5, 16, 22, 36):            # logical positions of sequence 0 (all cached)
        a = dict(arrays)
        a["q"] = arrays["q"].copy()
        key = arrays["k_cache"][tbl[0, target // BS], 0, target % BS, :].astype(np.float64)
        a["q"][0, :, :] = (400.0 * key / np.linalg.norm(key) ** 2).astype(np.float32)
        a["scale"] = 1.0
        _, _, _, _, out = run_oracle(orc, a)
        val = arrays["v_cache"][tbl[0, target // BS], 0, :, target % BS].astype(np.float64)
        for h in range(2):
            assert np.max(np.abs(out[0, h] - val)) < 1e-6, f"target {target} head {h}"


def pin_exact_weights(orc):
    """Closed form: one head, D=1, key_j = ln(j+1), q = 1, value_j = j  ->  out at p = 2p/3."""
    L = 45
    step = workload.build_step([0], [L], num_q_heads=1, num_kv_heads=1, head_dim=1, dtype="f32", seed=2)
    arrays = workload.host_arrays(step)
    a = dict(arrays)
    a["q"] = np.ones((L, 1, 1), dtype=np.float64)
    a["k"] = np.log(np.arange(1, L + 1, dtype=np.float64)).reshape(L, 1, 1)
    a["v"] = np.arange(L, dtype=np.float64).reshape(L, 1, 1)
    a["k_cache"] = arrays["k_cache"].astype(np.float64)
    a["v_cache"] = arrays["v_cache"].astype(np.float64)
    a["scale"] = 1.0
    _, _, _, _, out = run_oracle(orc, a)
    expect = 2.0 * np.arange(L) / 3.0
    err = np.max(np.abs(out[:, 0, 0] - expect))
    assert err <= 1e-12, f"closed form 2p/3: {err}"


def pin_slot_golden(orc):
    """Hand-worked slot-mapping example (tests/golden/slot_mapping_worked.json)."""
    with open(os.path.join(GOLDEN, "slot_mapping_worked.json")) as f:
        case = json.load(f)
    bt = np.full((len(case["block_tables"]), max(len(r) for r in case["block_tables"])), -1, np.int64)
    for i, row in enumerate(case["block_tables"]):
        bt[i, : len(row)] = row
    pos, slots = orc.slot_mapping(bt, np.asarray(case["query_start_loc"]), np.asarray(case["context_lens"]))
    assert pos.tolist() == case["positions"], (pos.tolist(), case["positions"])
    assert slots.tolist() == case["slots"], (slots.tolist(), case["slots"])


def pin_scatter_copy(orc, seeds=range(4)):
    """P5: the cache write copies each token's bits to its slot and leaves every other slot alone."""
    for seed in seeds:
        for dtype in ("f32", "bf16"):
            step = workload.build_step([3, 20, 0], [2, 1, 17], num_q_heads=4, num_kv_heads=2, head_dim=8,
                                       dtype=dtype, seed=seed, num_blocks=12)
            arrays = workload.host_arrays(step)
            slots = workload.random_slots(arrays["k"].shape[0], 12, pad_fraction=0.3, seed=seed)
            kc, vc = orc.reshape_and_cache(arrays["k"], arrays["v"], arrays["k_cache"], arrays["v_cache"], slots)
            expect_k, expect_v = arrays["k_cache"].copy(), arrays["v_cache"].copy()
            for t, s in enumerate(slots):
                if s < 0:
                    continue
                for g in range(2):
                    for dd in range(8):
                        expect_k[s // BS, g, s % BS, dd] = arrays["k"][t, g, dd]
                        expect_v[s // BS, g, dd, s % BS] = arrays["v"][t, g, dd]
            assert _bits_equal(kc, expect_k) and _bits_equal(vc, expect_v), f"seed {seed} {dtype}"


def pin_invariants(orc):
    """P4: paging and batching do not change any row's result."""
    # block placement and prefix sharing: bit-identical
    step, arrays = _step_arrays("prefix_shared_bf16")
    base = run_oracle(orc, arrays)[4]
    perm = run_oracle(orc, workload.host_arrays(workload.permute_blocks(step, seed=9)))[4]
    assert np.array_equal(base, perm, equal_nan=True), "block-id permutation changed the result"
    priv = run_oracle(orc, workload.host_arrays(workload.privatize_shared_prefix(step, seed=4)))[4]
    assert np.array_equal(base, priv, equal_nan=True), "private prefix copies changed the result"
    # sequence order and batch composition: each sequence's rows are unchanged
    step, arrays = _step_arrays("mixed_step_bf16")
    base = run_oracle(orc, arrays)[4]
    qsl = arrays["query_start_loc"]
    order = np.random.default_rng(3).permutation(step.num_seqs)
    shuf = run_oracle(orc, workload.host_arrays(workload.subset_sequences(step, order, compact_pool=False)))[4]
    rows = np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in order])
    assert np.array_equal(base[rows], shuf, equal_nan=True), "sequence order changed the result"
    for i in (0, step.num_seqs - 1):
        alone = run_oracle(orc, workload.host_arrays(workload.subset_sequences(step, [i])))[4]
        assert np.array_equal(base[qsl[i]:qsl[i + 1]], alone), f"sequence {i} alone differs from in batch"
    # chunk split: one chunk == two chunks over two steps (same keys, different grouping)
    full = workload.build_step([9], [40], num_q_heads=4, num_kv_heads=2, head_dim=16, dtype="bf16",
                               seed=6, num_blocks=6)
    farr = workload.host_arrays(full)
    _, _, kc_full, vc_full, out_full = run_oracle(orc, farr)
    cut = 23
    first = dict(farr)
    first.update(q=farr["q"][:cut], k=farr["k"][:cut], v=farr["v"][:cut],
                 seq_lens=np.array([9 + cut]), query_start_loc=np.array([0, cut]))
    _, _, kc1, vc1, out1 = run_oracle(orc, first)
    second = dict(farr)
    second.update(q=farr["q"][cut:], k=farr["k"][cut:], v=farr["v"][cut:], k_cache=kc1, v_cache=vc1,
                  context_lens=np.array([9 + cut]), query_start_loc=np.array([0, 40 - cut]))
    _, _, kc2, vc2, out2 = run_oracle(orc, second)
    assert _bits_equal(kc2, kc_full) and _bits_equal(vc2, vc_full), "chunked writes differ"
    err = np.max(np.abs(np.concatenate([out1, out2]) - out_full))
    assert err <= 1e-12, f"chunk split: {err}"
    # a decode row equals the last row of the same sequence run as one prefill chunk
    dec = dict(farr)
    dec.update(q=farr["q"][-1:], k=farr["k"][-1:], v=farr["v"][-1:], k_cache=kc2, v_cache=vc2,
               context_lens=np.array([48]), query_start_loc=np.array([0, 1]))
    # the decode step re-writes the same token's K/V into the same slot (same bits)
    out_dec = run_oracle(orc, dec)[4]
    err = np.max(np.abs(out_dec[0] - out_full[-1]))
    assert err <= 1e-12, f"decode row vs last prefill row: {err}"


def pin_rejects_bad_inputs(orc):
    """Preconditions are enforced (duplicate slots, inconsistent lengths, out-of-range ids)."""
    step, arrays = _step_arrays("tiny_decode_f32")
    ok = dict(arrays)

    def raises(**changes):
        a = dict(ok)
        a.update(changes)
        try:
            orc.validate_step(a["q"], a["k_cache"], a["v_cache"], a["block_tables"], a["seq_lens"],
                              a["query_start_loc"], a["context_lens"], slots=a.get("slots"))
        except orc.OracleInputError:
            return True
        return False

    assert not raises(), "valid input rejected"
    assert raises(slots=np.array([3, 3, 5, 7])), "duplicate slots accepted"
    assert raises(seq_lens=ok["seq_lens"] + 1), "inconsistent seq_lens accepted"
    bad_bt = ok["block_tables"].copy()
    bad_bt[3, 0] = 10_000
    assert raises(block_tables=bad_bt), "out-of-range block id accepted"
    assert raises(query_start_loc=np.array([0, 1, 1, 3, 4])), "query_start_loc inconsistent with lengths accepted"


ALL_PINS = [
    pin_bruteforce,
    pin_sdpa,
    pin_single_token,
    pin_constant_keys,
    pin_group_mapping,
    pin_aligned_query,
    pin_exact_weights,
    pin_slot_golden,
    pin_scatter_copy,
    pin_invariants,
    pin_rejects_bad_inputs,
]
