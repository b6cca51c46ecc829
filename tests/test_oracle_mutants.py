"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant edits one line of the oracle's source text (in memory, on the
CPU), loads the edited copy as a throw-away module and runs every pin against
it.  A mutant that passes all pins would mean the pins cannot see that kind of
mistake.
"""

import importlib.util
import os
import types

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "paged_decode.py")

MUTANTS = {
    "gqa_map_modulo": ("return h // group", "return h % num_kv_heads"),
    "scale_dropped": ("s = scale * (K @ q)", "s = (K @ q)"),
    "scale_inverted": ("s = scale * (K @ q)", "s = (K @ q) / scale"),
    "softmax_sign": ("e = np.exp(s - m)", "e = np.exp(m - s)"),
    "no_normalisation": ("o = (e @ V) / z", "o = (e @ V)"),
    "k_v_swapped": ("attention_one_query(q[h], K[:, g, :], V[:, g, :], scale)",
                    "attention_one_query(q[h], V[:, g, :], K[:, g, :], scale)"),
    "wrong_query_head": ("attention_one_query(q[h], K[:, g, :]",
                         "attention_one_query(q[g], K[:, g, :]"),
    "new_token_excluded": ("L = int(seq_lens[b])\n        if L == 0:\n            continue\n        K =",
                           "L = int(seq_lens[b]) - 1\n        if L <= 0:\n            continue\n        K ="),
    "tail_slots_read": ("valid = min(page_size, seq_len - i * page_size)", "valid = page_size"),
    "block_table_ignored": ("physical = int(block_table_row[i])", "physical = i"),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "lse_without_max": ("return o, w, m + math.log(z)", "return o, w, math.log(z)"),
    "weights_unnormalised": ("w = e / z", "w = e"),
    "append_slot_off_by_one": ("pos = L - 1", "pos = L"),
    "append_page_modulo": ("physical = int(block_tables[b][pos // page_size])",
                           "physical = int(block_tables[b][pos % page_size])"),
    "append_k_gets_v": ("k_out[physical, slot] = k_new_bits[b]",
                        "k_out[physical, slot] = v_new_bits[b]"),
    "fill_slot_off_by_one": ("t = start + j", "t = start + j + 1"),
    "fill_page_modulo": ("physical = int(block_table_row[t // page_size])",
                         "physical = int(block_table_row[t % page_size])"),
    "fill_v_gets_k": ("v_out[physical, t % page_size] = v_rows_bits[j]",
                      "v_out[physical, t % page_size] = k_rows_bits[j]"),
}


def _load_mutant(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mutant = _load_mutant(name, *MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # assertion or crash: either way the pin saw it
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name!r} passed every pin"


def test_unmutated_copy_passes():
    text = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(text, "<copy>", "exec"), mod.__dict__)
    for pin in ALL_PINS:
        pin(mod)
