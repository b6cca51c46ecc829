"""The reference allocator against its pins; planted mistakes against the pins."""

import os
import types

import pytest

from oracle import admission
from oracle_pins_admission import ALL_ADMISSION_PINS

SRC = admission.__file__


@pytest.mark.parametrize("pin", ALL_ADMISSION_PINS, ids=lambda f: f.__name__)
def test_admission_pin(pin):
    pin(admission)


MUTANTS = {
    "credit_without_minus_one": ("self.pages_for(prompt + allowed_new - 1)",
                                 "self.pages_for(prompt + allowed_new)"),
    "credit_one_layer": ("return allowed_new, self.layers * self.pages_for",
                         "return allowed_new, self.pages_for"),
    "no_context_cap": ("allowed_new = min(max_new, self.context - prompt)",
                       "allowed_new = max_new"),
    "overtaking": ("                if self.reserved + r.credit > self.num_pages:\n                    break",
                   "                if self.reserved + r.credit > self.num_pages:\n                    self.waiting.rotate(-1)\n                    if all(self.reserved + x.credit > self.num_pages for x in self.waiting):\n                        break\n                    continue"),
    "finish_keeps_credit": ("        self.reserved -= r.credit\n", "\n"),
    "static_ignored": ("if not (self.static and self.active):", "if True:"),
    "no_reject_when_too_big": ("        if credit > self.num_pages:\n            return REJECT\n", "\n"),
    "highest_free_page": ("r.pages[layer].append(heapq.heappop(self.free))",
                          "r.pages[layer].append(self.free.pop(self.free.index(max(self.free))))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_admission_mutant_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, name
    mod = types.ModuleType(f"admission_mutant_{name}")
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = 0
    for pin in ALL_ADMISSION_PINS:
        try:
            pin(mod)
        except Exception:
            caught += 1
    assert caught, f"planted mistake {name!r} passed every pin"
