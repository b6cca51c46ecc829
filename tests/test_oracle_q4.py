"""The INT4 K/V page oracle against its pins, and planted mistakes against the pins."""

import os
import types

import pytest

import oracle
from oracle import kvquant
from oracle_pins_q4 import ALL_Q4_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvquant.py")


@pytest.mark.parametrize("pin", ALL_Q4_PINS, ids=lambda f: f.__name__)
def test_q4_pin(pin):
    pin(kvquant)


MUTANTS = {
    "store_offset_7": ("u = (np.asarray(codes, np.int16) + 8)", "u = (np.asarray(codes, np.int16) + 7)"),
    "nibbles_swapped": ("return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)",
                        "return (u[..., 1::2] | (u[..., 0::2] << 4)).astype(np.uint8)"),
    "read_offset_7": ("out[..., 0::2] = (b & 0x0F).astype(np.int16) - 8",
                      "out[..., 0::2] = (b & 0x0F).astype(np.int16) - 7"),
    "divide_by_8": ("QMAX4 = 7 ", "QMAX4 = 8 "),
    "int8_range_for_int4": ("qmax, qmin = (QMAX, QMIN) if nbits == 8 else (QMAX4, QMIN4)",
                            "qmax, qmin = (QMAX, QMIN)"),
    "codes_not_packed": ("        kc, vc = pack_q4(kc), pack_q4(vc)\n", "        pass\n"),
    "high_nibble_sign": ("out[..., 1::2] = (b >> 4).astype(np.int16) - 8",
                         "out[..., 1::2] = (b >> 4).astype(np.int16) - 8 * (b >> 7)"),
}


def _mutant(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, name
    text = text.replace(old, new).replace("from .paged_decode import", "from oracle.paged_decode import")
    mod = types.ModuleType(f"kvquant_q4_mutant_{name}")
    exec(compile(text, f"<kvquant q4 mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_q4_mutant_is_caught(name):
    m = _mutant(name, *MUTANTS[name])
    caught = []
    for pin in ALL_Q4_PINS:
        try:
            pin(m)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name!r} passed every INT4 pin"
