"""The oracle's RoPE step against its pins, and planted mistakes against the pins."""

import os
import types

import pytest

import oracle
from oracle import rope
from oracle_pins_rope import ALL_ROPE_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "rope.py")


@pytest.mark.parametrize("pin", ALL_ROPE_PINS, ids=lambda f: f.__name__)
def test_rope_pin(pin):
    pin(rope)


MUTANTS = {
    "interleaved_pairs": ("x1, x2 = x[..., :half], x[..., half:]",
                          "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    "sin_sign": ("a = (x1 * c).astype(np.float32) - (x2 * s).astype(np.float32)",
                 "a = (x1 * c).astype(np.float32) + (x2 * s).astype(np.float32)"),
    "position_L": ("pos = L - 1", "pos = min(L, len(rope_cos) - 1)"),
    "truncating_round": ("up = (low > half) | ((low == half) & ((down & 1) == 1))",
                         "up = low < 0"),
    "ties_away": ("up = (low > half) | ((low == half) & ((down & 1) == 1))",
                  "up = low >= half"),
    "k_not_rotated": ("k_out[b] = f32_to_bf16_bits_rne(rope_rotate_f32(k_new_bits[b], rope_cos[pos], rope_sin[pos]))",
                      "k_out[b] = k_new_bits[b]"),
}


def _mutant(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, name
    text = text.replace(old, new).replace("from .paged_decode import", "from oracle.paged_decode import")
    mod = types.ModuleType(f"rope_mutant_{name}")
    exec(compile(text, f"<rope mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rope_mutant_is_caught(name):
    m = _mutant(name, *MUTANTS[name])
    caught = 0
    for pin in ALL_ROPE_PINS:
        try:
            pin(m)
        except Exception:
            caught += 1
    assert caught, f"planted mistake {name!r} passed every RoPE pin"
