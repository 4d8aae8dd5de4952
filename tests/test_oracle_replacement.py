"""Pins of the oracle's circular and clock replacement policies.

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "GPU cache management has hazards too": the first GPU hot cache used
clock replacement with reference bits, which was pathological on a probe with
a full hot cache, all reference bits set and 1% misses; it was replaced by
circular eviction that skips the slots pinned by the current round.

Readings (the pages name the policies but do not define them): misses are
served one at a time in ascending position order.  Circular: a hand moves
over the slots and takes the next slot not used in the current step.  Clock:
hits and fills set a slot's reference bit; the hand skips slots used in the
current step, clears and skips set bits, and takes the first slot with a
clear bit.  Both hands start at slot 0 and stop just past their last victim.

Pins, none of which reuses the oracle's code:
  * independent Python implementations (slot records and an explicit hand)
    on random runs: victims, evictions, slot maps, reference bits, hand;
  * closed forms: a cold cache fills slots 0, 1, 2, ... in miss order; the
    page's probe (full cache, all bits set, m misses) gives as victims the
    first m unpinned slots from the hand, and leaves every other unpinned
    slot's bit clear; pinned slots are never victims; refilling every slot
    each step, clock takes the same victims as circular.
"""
import numpy as np
import pytest

import oracle


class PyHand:
    """Independent reference for the circular and clock policies."""

    def __init__(self, slots, clock):
        self.C, self.clock = slots, clock
        self.pos = [None] * slots
        self.last = [-1] * slots
        self.ref = [0] * slots
        self.hand = 0

    def victim(self, t):
        for _ in range(2 * self.C):
            v = self.hand
            self.hand = (self.hand + 1) % self.C
            if self.last[v] == t:
                continue
            if self.clock and self.ref[v]:
                self.ref[v] = 0
                continue
            return v
        raise AssertionError("no victim")

    def step(self, t, sel):
        where = {p: v for v, p in enumerate(self.pos) if p is not None}
        for p in sel:
            if p in where:
                self.last[where[p]] = t
                self.ref[where[p]] = 1
        events = []
        for p in sel:
            if p in where:
                continue
            v = self.victim(t)
            old = self.pos[v]
            events.append((p, v, -1 if old is None else old))
            if old is not None:
                del where[old]
            self.pos[v], self.last[v], self.ref[v] = p, t, 1
            where[p] = v
        return events


def _stream(rng, h, k, steps):
    hot = rng.choice(h, size=3 * k, replace=False)
    out = []
    for _ in range(steps):
        pool = hot if rng.random() < 0.7 else np.arange(h)
        out.append(np.sort(rng.choice(pool, size=k, replace=False)).astype(np.int32))
    return out


@pytest.mark.parametrize("policy", [oracle.CIRCULAR, oracle.CLOCK])
@pytest.mark.parametrize("seed", range(6))
def test_against_python_reference(policy, seed):
    rng = np.random.default_rng(100 + seed)
    H, K = 400, int(rng.integers(4, 40))
    C = K + int(rng.integers(0, 60))
    rows = rng.integers(0, 256, (H, 656), dtype=np.uint8)
    c = oracle.Cache(C, H, policy)
    ref = PyHand(C, policy == oracle.CLOCK)
    for t, sel in enumerate(_stream(rng, H, K, 25)):
        info = c.step(t, sel, rows)
        ev = ref.step(t, [int(p) for p in sel])
        m = info["n_miss"]
        assert m == len(ev)
        np.testing.assert_array_equal(info["miss_pos"][:m], [e[0] for e in ev])
        np.testing.assert_array_equal(info["victim"][:m], [e[1] for e in ev])
        np.testing.assert_array_equal(info["evicted"][:m], [e[2] for e in ev])
        np.testing.assert_array_equal(c.pos_of(), [-1 if p is None else p for p in ref.pos])
        np.testing.assert_array_equal(c.last(), ref.last)
        assert c.hand() == ref.hand
        if policy == oracle.CLOCK:
            np.testing.assert_array_equal(c.ref(), ref.ref)
        res = np.flatnonzero(c.pos_of() >= 0)
        np.testing.assert_array_equal(c.hot()[res], rows[c.pos_of()[res]])
    c.close()


@pytest.mark.parametrize("policy", [oracle.CIRCULAR, oracle.CLOCK])
def test_cold_fill_takes_slots_in_order(policy):
    H, K, C = 1000, 50, 200
    rows = np.zeros((H, 656), np.uint8)
    c = oracle.Cache(C, H, policy)
    for t in range(4):
        sel = np.arange(t * K, (t + 1) * K, dtype=np.int32)
        info = c.step(t, sel, rows)
        np.testing.assert_array_equal(info["victim"][:K], np.arange(t * K, (t + 1) * K))
        assert info["n_evict"] == 0
    assert c.hand() == 0           # 4 x 50 = 200 slots: the hand wrapped to slot 0
    c.close()


def _full_cache(policy, C, K):
    """Cache of C slots filled by C / K steps of disjoint selections."""
    H = 4 * C
    rows = np.zeros((H, 656), np.uint8)
    c = oracle.Cache(C, H, policy)
    for t in range(C // K):
        c.step(t, np.arange(t * K, (t + 1) * K, dtype=np.int32), rows)
    return c, rows, C // K


@pytest.mark.parametrize("policy", [oracle.CIRCULAR, oracle.CLOCK])
def test_page_probe_full_cache_all_bits_set_one_percent_misses(policy):
    C, K = 2048, 256
    c, rows, t = _full_cache(policy, C, K)
    if policy == oracle.CLOCK:
        assert c.ref().all()       # every slot was filled, so every bit is set
    hand0 = c.hand()
    rng = np.random.default_rng(5)
    old = np.sort(rng.choice(C, size=K - 3, replace=False))  # resident positions = slots
    new = np.array([C + 1, C + 2, C + 3])
    sel = np.sort(np.concatenate([old, new])).astype(np.int32)
    pinned = set(int(c.slot_of()[p]) for p in old)
    info = c.step(t, sel, rows)
    order = [(hand0 + i) % C for i in range(C)]
    free = [v for v in order if v not in pinned]
    np.testing.assert_array_equal(info["victim"][:3], free[:3])
    if policy == oracle.CLOCK:
        r = c.ref()
        assert all(r[v] == 0 for v in free[3:])      # one revolution cleared them
        assert all(r[v] == 1 for v in pinned) and all(r[v] == 1 for v in free[:3])
    c.close()


def test_clock_refilling_every_slot_walks_like_circular():
    """With C = K and fresh positions every step, every slot is refilled each
    step: clock's first revolution clears every bit, after which it takes the
    slots in the same order as circular."""
    H, K = 5000, 64
    rows = np.zeros((H, 656), np.uint8)
    a, b = oracle.Cache(K, H, oracle.CIRCULAR), oracle.Cache(K, H, oracle.CLOCK)
    for t in range(10):
        sel = np.arange(t * K, (t + 1) * K, dtype=np.int32)
        ia, ib = a.step(t, sel, rows), b.step(t, sel, rows)
        np.testing.assert_array_equal(ia["victim"], ib["victim"])
    a.close()
    b.close()


@pytest.mark.parametrize("policy", [oracle.CIRCULAR, oracle.CLOCK])
def test_pinned_slots_are_never_victims(policy):
    rng = np.random.default_rng(9)
    H, K, C = 600, 40, 48
    rows = np.zeros((H, 656), np.uint8)
    c = oracle.Cache(C, H, policy)
    for t in range(40):
        sel = np.sort(rng.choice(H, K, replace=False)).astype(np.int32)
        before = c.slot_of()
        pinned = {int(before[p]) for p in sel if before[p] >= 0}
        info = c.step(t, sel, rows)
        assert not pinned & set(info["victim"][:info["n_miss"]].tolist())
        assert np.all(c.slot_of()[sel] >= 0)
    c.close()
