"""The C++ page allocator (include/pa_kvpool.h) against the reference model.

No GPU: the allocator is host code.  The black-box pins of the reference run
against the C++ pool through a small adapter, and random request traces are
replayed on both, comparing every result, every block table and the counters.
"""

import types

import numpy as np
import pytest

from oracle import admission as ref
from oracle_pins_admission import ALL_ADMISSION_PINS
from paged_kv_decode_07_amd import binding as pa


class _Active(dict):
    pass


def _cpp_module():
    """A module-like adapter exposing PagePool/WAIT/REJECT over the C++ pool."""

    class PagePool:
        def __init__(self, num_pages, num_layers=16, page_tokens=16, context=2048, static=False):
            self._p = pa.KVPool(num_pages, num_layers, page_tokens, context, static)
            self.num_pages = num_pages

        def credit_for(self, prompt, max_new):
            return self._p.credit_for(prompt, max_new)

        def submit(self, rid, prompt, max_new):
            return self._p.submit(rid, prompt, max_new)

        def admit(self):
            return self._p.admit()

        def grow(self, rid, length):
            self._p.grow(rid, length)

        def step(self):
            self._p.step()

        def finish(self, rid):
            self._p.finish(rid)

        def block_table(self, rid, layer):
            return self._p.block_table(rid, layer)

        @property
        def stats(self):
            return self._p.stats

    return types.SimpleNamespace(PagePool=PagePool, WAIT=ref.WAIT, REJECT=ref.REJECT)


BLACK_BOX = [p for p in ALL_ADMISSION_PINS if p.__name__ != "pin_random_trace_invariants"]


@pytest.mark.parametrize("pin", BLACK_BOX, ids=lambda f: f.__name__)
def test_cpp_pool_passes_reference_pins(pin):
    pin(_cpp_module())


@pytest.mark.parametrize("seed,static", [(1, False), (2, False), (3, True), (4, False)])
def test_cpp_pool_matches_reference_on_random_traces(seed, static):
    rng = np.random.default_rng(seed)
    layers = int(rng.integers(1, 5))
    pages = int(rng.integers(50, 600))
    a = ref.PagePool(pages, num_layers=layers, context=512, static=static)
    b = pa.KVPool(pages, layers, 16, 512, static)
    next_id, live = 0, []
    for _ in range(1500):
        op = int(rng.integers(0, 5))
        if op == 0:
            prompt, mx = int(rng.integers(0, 520)), int(rng.integers(0, 300))
            assert a.submit(next_id, prompt, mx) == b.submit(next_id, prompt, mx)
            next_id += 1
        elif op == 1:
            got = b.admit()
            assert got == a.admit()
            for rid in got:
                prompt = a.active[rid].prompt
                a.grow(rid, prompt); b.grow(rid, prompt)
                live.append(rid)
        elif op in (2, 3) and live:
            rid = live[int(rng.integers(0, len(live)))]
            r = a.active[rid]
            top = r.prompt + r.allowed_new - 1
            L = min(top, r.length + int(rng.integers(1, 40)))
            a.grow(rid, L); b.grow(rid, L)
            a.step(); b.step()
            info = b.info(rid)
            assert (info["allowed_new"], info["credit"], info["length"]) == \
                (r.allowed_new, r.credit, r.length)
        elif op == 4 and live:
            rid = live.pop(int(rng.integers(0, len(live))))
            a.finish(rid); b.finish(rid)
        for rid in live:
            for layer in range(layers):
                assert b.block_table(rid, layer, 64) == a.block_table(rid, layer)
        assert b.stats == a.stats


def test_cpp_pool_errors():
    p = pa.KVPool(32, 2, 16, 256)
    with pytest.raises(RuntimeError):
        p.grow(7, 3)                                  # unknown request
    assert p.submit(1, 10, 5) == "wait"
    with pytest.raises(RuntimeError):
        p.submit(1, 10, 5)                            # id in use
    assert p.admit() == [1]
    with pytest.raises(RuntimeError):
        p.grow(1, 15)                                 # beyond prompt + allowed - 1 = 14
    p.grow(1, 14)
    with pytest.raises(RuntimeError):
        p.grow(1, 3)                                  # lengths never shrink
    with pytest.raises(RuntimeError):
        p.block_table(1, 2)                           # no such layer
    p.submit(2, 10, 5)
    with pytest.raises(RuntimeError):
        p.admit(capacity=0)                           # array too small: nothing admitted
    assert p.admit() == [2]
    p.finish(1)
    with pytest.raises(RuntimeError):
        p.finish(1)
