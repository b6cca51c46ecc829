"""The INT8 K/V page oracle against its pins, and planted mistakes against the pins."""

import os
import types

import pytest

import oracle
from oracle import kvquant
from oracle_pins_kvquant import ALL_KVQUANT_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvquant.py")


@pytest.mark.parametrize("pin", ALL_KVQUANT_PINS, ids=lambda f: f.__name__)
def test_kvquant_pin(pin):
    pin(kvquant)


MUTANTS = {
    "divide_by_qmax_plus_one": ("scale = (amax / np.float32(qmax))", "scale = (amax / np.float32(qmax + 1))"),
    "one_scale_per_tensor": ("amax = np.max(np.abs(x), axis=-1)",
                             "amax = np.max(np.abs(x), axis=-1) * 0 + np.max(np.abs(x))"),
    "truncating_round": ("codes = np.clip(np.rint(ratio), qmin, qmax)",
                         "codes = np.clip(np.trunc(ratio), qmin, qmax)"),
    "ties_up": ("codes = np.clip(np.rint(ratio), qmin, qmax)",
                "codes = np.clip(np.floor(ratio + np.float32(0.5)), qmin, qmax)"),
    "multiply_by_scale": ("ratio = (x / safe[..., None])", "ratio = (x * safe[..., None])"),
    "v_scale_into_k_slot": ("scales[physical, :, 1, slot] = vs", "scales[physical, :, 0, slot] = vs"),
    "scale_slot_wrong": ("scales[physical, :, 0, slot] = ks", "scales[physical, :, 0, 0] = ks"),
    "k_codes_not_written": ("    k_codes[physical, :, slot] = kc\n", "    pass\n"),
    "gather_k_scale_for_v": ("rows.append(dequantize(c, scales[physical, :, which, slot]))",
                             "rows.append(dequantize(c, scales[physical, :, 0, slot]))"),
    "dequantize_without_scale": ("return np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[..., None]",
                                 "return np.asarray(codes, np.float64)"),
    "append_slot_off_by_one": ("_write_token(kc, vc, sc, physical, pos % page_size,",
                               "_write_token(kc, vc, sc, physical, (pos + 1) % page_size,"),
    "bound_without_value_term": ("return grow * (w @ np.abs(V_hat)) + w @ np.abs(V_hat - V)",
                                 "return grow * (w @ np.abs(V_hat))"),
    "bound_without_weight_term": ("return grow * (w @ np.abs(V_hat)) + w @ np.abs(V_hat - V)",
                                  "return w @ np.abs(V_hat - V)"),
    "bound_single_eps": ("grow = math.expm1(2.0 * eps)", "grow = math.expm1(0.5 * eps)"),
}


def _mutant(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, name
    text = text.replace(old, new).replace("from .paged_decode import", "from oracle.paged_decode import")
    mod = types.ModuleType(f"kvquant_mutant_{name}")
    exec(compile(text, f"<kvquant mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_kvquant_mutant_is_caught(name):
    m = _mutant(name, *MUTANTS[name])
    caught = []
    for pin in ALL_KVQUANT_PINS:
        try:
            pin(m)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"planted mistake {name!r} passed every INT8 pin"
