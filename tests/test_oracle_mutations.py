"""Plant plausible mistakes in a copy of the oracle; some pin must catch each one.

Each mutant is the oracle's source with one textual change (an off-by-one mask, a
dropped term, a swapped index, a transposed operand ...), executed as a fresh module.
The real oracle module is never modified.
"""

import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "paged_attention.py")

MUTATIONS = {
    "mask_off_by_one": ("<= pos[:, None]", "< pos[:, None]"),
    "group_strided": ("heads = slice(g * group, (g + 1) * group)", "heads = slice(g, hq, hkv)"),
    "dropped_scale": ("scores = scale * (qg @ keys[:, g, :].T)", "scores = (qg @ keys[:, g, :].T)"),
    "softmax_sign": ("np.exp(scores - peak)", "np.exp(peak - scores)"),
    "dropped_context_in_slots": ("p = int(ctx[i]) + (t - int(qsl[i]))", "p = (t - int(qsl[i]))"),
    "dropped_context_in_positions": ("pos = ctx[i] + r_sel", "pos = r_sel"),
    "slot_offset": ("* BLOCK_SIZE + p % BLOCK_SIZE", "* BLOCK_SIZE + (p + 1) % BLOCK_SIZE"),
    "value_layout_transposed": ("vals = vb.transpose(0, 3, 1, 2)", "vals = vb.transpose(0, 3, 1, 2)[:, ::-1]"),
    "key_block_offset": ("keys = kb.transpose(0, 2, 1, 3)", "keys = kb.transpose(0, 2, 1, 3)[:, ::-1]"),
    "scatter_value_transposed": ("new_v[b, :, :, o] = v[t]", "new_v[b, :, :, BLOCK_SIZE - 1 - o] = v[t]"),
    "normaliser_global": ("/ weights.sum(axis=1, keepdims=True)", "/ weights.sum()"),
    "bf16_widen_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "gqa_kv_index": ("scores = scale * (qg @ keys[:, g, :].T)", "scores = scale * (qg @ keys[:, 0, :].T)"),
    "values_from_keys": ("o = (weights @ vals[:, g, :])", "o = (weights @ keys[:, g, :])"),
    "skip_padding_wrong": ("if s < 0:\n            continue", "if s < -1:\n            continue"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation {name}: pattern not found in the oracle source"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(name)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # a failed assertion or a crash both count as caught
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
    assert caught, f"no pin caught mutation {name}"
