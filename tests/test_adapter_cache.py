"""The adapter cache's host policy (no GPU): which slots and pages a batch's missing adapters
get, whom they evict, and what every load must wait for.  The GPU side (loads, events) is in
tests/test_gpu_adapter_cache.py."""
import types

import numpy as np
import pytest

from segmented_gather_matmul_amd import binding as B
from segmented_gather_matmul_amd.adapters import AdapterCache


def _cache(num_slots, num_pages, pages_of):
    """A cache over a stand-in model (slot count and a free-page list only) and a store
    whose adapters take pages_of[key] pages (split over two targets)."""
    model = types.SimpleNamespace(num_slots=num_slots, state=B.PoolState(num_pages))
    store = {k: types.SimpleNamespace(n_pages=[n // 2, n - n // 2]) for k, n in pages_of.items()}
    return AdapterCache(model, store, streams=[object()])


def _apply(c, keys, used=None):
    """plan + take for a batch, as ensure does minus the GPU; returns the plan and the waits."""
    steps = c.plan(keys)
    waits = []
    for k, slot, evicted in steps:
        _, w = c.take(k, slot, evicted)
        waits.append(w)
    for k in keys:
        if k is not None:
            c.lru.move_to_end(k)
    if used is not None:
        for k in set(k for k in keys if k is not None):
            c.last_use[c.slot_of[k]] = used
    return steps, waits


def _invariants(c, num_pages):
    slots = list(c.slot_of.values())
    assert len(slots) == len(set(slots))
    for k, s in c.slot_of.items():
        assert c.key_in[s] == k
    assert sum(k is not None for k in c.key_in) == len(c.slot_of)
    assert list(c.lru) == [k for k in c.lru if k in c.slot_of] and set(c.lru) == set(c.slot_of)
    taken = np.concatenate(list(c.pages.values())) if c.pages else np.zeros(0, np.int32)
    assert len(taken) == len(set(taken.tolist()))                       # no page in two adapters
    assert c.model.state.free == num_pages - len(taken)


def test_fill_then_evict_least_recently_used():
    c = _cache(3, 100, {k: 10 for k in "abcdef"})
    steps, _ = _apply(c, ["a", "b", None, "a"])
    assert [(k, s) for k, s, _ in steps] == [("a", 0), ("b", 1)] and all(not e for _, _, e in steps)
    _apply(c, ["c"])
    _invariants(c, 100)
    _apply(c, ["a"])                                  # a becomes the most recent
    steps, _ = _apply(c, ["d", "a"])                  # evicts b (least recent), not a
    assert steps == [("d", 1, ["b"])]
    assert set(c.slot_of) == {"a", "c", "d"}
    _invariants(c, 100)


def test_batch_keys_are_never_evicted():
    c = _cache(2, 100, {k: 10 for k in "abc"})
    _apply(c, ["a", "b"])
    with pytest.raises(ValueError, match="3 distinct adapters in one batch, 2 slots"):
        c.plan(["a", "b", "c"])
    steps, _ = _apply(c, ["b", "c"])                  # a goes, b stays
    assert steps == [("c", 0, ["a"])]
    _invariants(c, 100)


def test_page_pressure_evicts_more_than_the_slot():
    # 4 slots but pages for only about 3 adapters of 30 pages
    c = _cache(4, 95, {"a": 30, "b": 30, "c": 30, "d": 30, "e": 10})
    _apply(c, ["a", "b", "c"])
    steps, _ = _apply(c, ["d"])                       # a free slot, but no pages: evict a
    assert steps == [("d", 3, ["a"])]
    _invariants(c, 95)
    with pytest.raises(ValueError, match="no room"):
        c.plan(["e", "b", "c", "d"])                  # 5 pages free, nothing the batch may evict
    steps, _ = _apply(c, ["e", "b", "c"])             # a's slot is free; d goes for its pages
    assert steps == [("e", 0, ["d"])]
    assert c.key_in[3] is None
    _invariants(c, 95)


def test_loads_wait_for_the_last_readers_of_what_they_reuse():
    c = _cache(2, 40, {k: 20 for k in "abc"})
    e1, e2 = object(), object()
    _apply(c, ["a"], used=e1)
    _apply(c, ["b"], used=e2)
    steps, waits = _apply(c, ["c"])                   # evicts a: its slot and its pages
    assert steps == [("c", 0, ["a"])] and waits == [[e1]]
    # pages released in order come back as the same run
    assert np.array_equal(c.pages["c"], np.arange(20))


def test_unknown_key():
    c = _cache(2, 40, {"a": 10})
    with pytest.raises(KeyError):
        c.plan(["zz"])
