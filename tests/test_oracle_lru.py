"""Pins of the oracle's hot-cache replacement (LRU by last-use step).

The hot cache is a bounded slot array (page "From 1M Total to 15+ × 1M
Contexts: GLM-5.3 KV Cache Offloading", section "Decision three: let the GPU
manage the hot cache directly"); slots used by the current round may not be
replaced (section "GPU cache management has hazards too").  Replacement:
the victim is the slot with the oldest last-use step, ties to the lowest slot;
an empty slot counts as used at step -1; misses are served in ascending
position order, one victim each.

Pins, none of which reuses the oracle's code:
  * an independent pure-Python LRU (records + min()) on random tiny runs;
  * closed forms: cold fill puts miss i in slot i; no eviction while the union
    of selections fits; C == K leaves exactly the current selection; a
    repeated selection misses only on its first step;
  * invariants after every step, including the step-granular stack property
    and inclusion between two capacities over one stream (the README of
    vllm-bounded-fs-kv-tier, section on sizing the tier: an LRU with fewer
    slots fed the same stream holds a subset of a larger one).
"""
import numpy as np
import pytest

import oracle


class PyLRU:
    """Independent reference: a list of slot records and min() per miss."""

    def __init__(self, slots):
        self.recs = [{"slot": v, "pos": None, "last": -1} for v in range(slots)]

    def step(self, t, sel):
        resident = {r["pos"]: r for r in self.recs if r["pos"] is not None}
        for p in sel:
            if p in resident:
                resident[p]["last"] = t
        events = []
        for p in sel:
            if p in resident:
                continue
            r = min((r for r in self.recs if r["last"] != t),
                    key=lambda r: (r["last"], r["slot"]))
            events.append((p, r["slot"], -1 if r["pos"] is None else r["pos"]))
            r["pos"], r["last"] = p, t
        return events

    def slot_of(self, p):
        for r in self.recs:
            if r["pos"] == p:
                return r["slot"]
        return -1


def random_stream(rng, h, k, steps, locality):
    """Selections of k distinct positions of [0, h), ascending."""
    hot = rng.choice(h, size=min(h, 3 * k), replace=False)
    out = []
    for _ in range(steps):
        if rng.random() < locality:
            pool = hot
        else:
            pool = np.arange(h)
        sel = np.sort(rng.choice(pool, size=k, replace=False)).astype(np.int32)
        out.append(sel)
    return out


def rows_for(h, seed=0):
    return np.random.default_rng(seed).integers(0, 256, (h, 656), dtype=np.uint8)


def check_invariants(c, t, sel, info, rows, used_at, occupancy_before):
    slot_of, pos_of, last, hot = c.slot_of(), c.pos_of(), c.last(), c.hot()
    # every selected position is resident and was used at t
    assert np.all(slot_of[sel] >= 0)
    assert np.all(last[slot_of[sel]] == t)
    # maps are mutual inverses; occupancy bounded by C
    res = np.flatnonzero(pos_of >= 0)
    assert res.size <= c.C
    np.testing.assert_array_equal(slot_of[pos_of[res]], res)
    assert (slot_of >= 0).sum() == res.size
    # victims: distinct, never a slot used at t before its fill
    m = info["n_miss"]
    v = info["victim"][:m]
    assert np.unique(v).size == m
    assert np.all(np.isin(v, info["slot"]))
    hits = info["slot"][np.isin(sel, info["miss_pos"][:m], invert=True)]
    assert not np.intersect1d(v, hits).size
    # evictions = misses beyond the free slots
    free = c.C - occupancy_before
    assert info["n_evict"] == max(0, m - free)
    # resident bytes equal the host rows
    np.testing.assert_array_equal(hot[res], rows[pos_of[res]])
    # stack property: everything used after t* resident, nothing used before
    used = np.flatnonzero(used_at >= 0)
    resident = np.zeros(used_at.size, bool)
    resident[pos_of[res]] = True
    if (~resident[used]).any():
        assert used_at[used[~resident[used]]].max() <= used_at[pos_of[res]].min()


@pytest.mark.parametrize("seed", range(30))
def test_against_python_lru(seed):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, 9))
    C = int(rng.choice([k, k + 1, 2 * k, 4 * k]))
    h = int(rng.integers(k, 65))
    steps = int(rng.integers(1, 51))
    rows = rows_for(h, seed)
    c, ref = oracle.Cache(C, h), PyLRU(C)
    used_at = np.full(h, -1)
    for t, sel in enumerate(random_stream(rng, h, k, steps, 0.6)):
        occ = (c.pos_of() >= 0).sum()
        info = c.step(t, sel, rows)
        used_at[sel] = t
        ev = ref.step(t, [int(p) for p in sel])
        m = info["n_miss"]
        assert m == len(ev)
        np.testing.assert_array_equal(info["miss_pos"][:m], [e[0] for e in ev])
        np.testing.assert_array_equal(info["victim"][:m], [e[1] for e in ev])
        np.testing.assert_array_equal(info["evicted"][:m], [e[2] for e in ev])
        np.testing.assert_array_equal(info["slot"], [ref.slot_of(int(p)) for p in sel])
        assert np.all(info["miss_pos"][m:] == -1)
        check_invariants(c, t, sel, info, rows, used_at, occ)


def test_cold_fill_puts_miss_i_in_slot_i():
    rows = rows_for(100)
    c = oracle.Cache(64, 100)
    sel = np.array([3, 7, 8, 20, 50, 99], np.int32)
    info = c.step(0, sel, rows)
    assert info["n_miss"] == 6 and info["n_hit"] == 0 and info["n_evict"] == 0
    np.testing.assert_array_equal(info["victim"][:6], np.arange(6))
    np.testing.assert_array_equal(info["slot"], np.arange(6))


@pytest.mark.parametrize("seed", range(5))
def test_no_eviction_while_the_union_fits(seed):
    rng = np.random.default_rng(50 + seed)
    h, k, C = 400, 16, 128
    rows = rows_for(h, seed)
    c = oracle.Cache(C, h)
    seen = set()
    for t, sel in enumerate(random_stream(rng, h, k, 40, 0.8)):
        new = set(sel.tolist()) - seen
        if len(seen | new) > C:
            break
        info = c.step(t, sel, rows)
        assert info["n_miss"] == len(new)
        assert info["n_evict"] == 0
        # fills go to slots in order of first appearance
        np.testing.assert_array_equal(info["victim"][:len(new)],
                                      np.arange(len(seen), len(seen) + len(new)))
        seen |= new


@pytest.mark.parametrize("seed", range(10))
def test_used_slots_are_a_prefix_and_fill_before_evicting(seed):
    """No slot ever becomes empty again and an empty slot (last use -1) is
    older than any used one, lowest slot first: after every step the used
    slots are exactly [0, fill), and the step that runs out of empty slots
    takes fill .. C - 1 first (evicting nothing) and evicts only for the
    misses beyond them.  C is not a multiple of K, so that step is mixed."""
    rng = np.random.default_rng(300 + seed)
    k = int(rng.integers(3, 20))
    C = k + int(rng.integers(1, 3 * k))
    if C % k == 0:
        C += 1
    h = int(rng.integers(4 * C, 8 * C))
    rows = rows_for(h, seed)
    c = oracle.Cache(C, h)
    fill, mixed = 0, 0
    for t, sel in enumerate(random_stream(rng, h, k, 30, 0.3)):
        info = c.step(t, sel, rows)
        m = info["n_miss"]
        n_new = min(m, C - fill)
        np.testing.assert_array_equal(info["victim"][:n_new], np.arange(fill, fill + n_new))
        assert np.all(info["evicted"][:n_new] == -1)
        assert np.all(info["evicted"][n_new:m] >= 0)
        assert info["n_evict"] == m - n_new
        mixed += 0 < n_new < m
        fill += n_new
        last = c.last()
        assert np.all(last[:fill] >= 0) and np.all(last[fill:] == -1)
    assert fill == C and mixed == 1
    c.close()


def test_capacity_equal_k_holds_exactly_the_current_selection():
    rng = np.random.default_rng(9)
    h, k = 60, 8
    rows = rows_for(h)
    c = oracle.Cache(k, h)
    for t, sel in enumerate(random_stream(rng, h, k, 30, 0.5)):
        c.step(t, sel, rows)
        res = np.sort(c.pos_of())
        np.testing.assert_array_equal(res, sel)


def test_repeated_selection_misses_only_once():
    rows = rows_for(500)
    c = oracle.Cache(300, 500)
    sel = np.arange(0, 500, 2, dtype=np.int32)[:200]
    for t in range(5):
        info = c.step(t, sel, rows)
        assert info["n_miss"] == (200 if t == 0 else 0)
        assert info["n_hit"] == (0 if t == 0 else 200)


def test_lru_order_and_pinning_worked_example():
    # C = 4, K = 2, worked by hand.
    rows = rows_for(10)
    c = oracle.Cache(4, 10)
    i0 = c.step(0, np.array([1, 2], np.int32), rows)   # slots 0,1 <- 1,2
    i1 = c.step(1, np.array([3, 4], np.int32), rows)   # slots 2,3 <- 3,4
    i2 = c.step(2, np.array([2, 5], np.int32), rows)   # hit 2 (slot 1); 5 evicts slot 0 (pos 1)
    i3 = c.step(3, np.array([6, 7], np.int32), rows)   # oldest: slots 2,3 (last 1)
    i4 = c.step(4, np.array([1, 6], np.int32), rows)   # hit 6; 1 takes the oldest, lowest slot
    assert list(i0["victim"][:2]) == [0, 1]
    assert list(i1["victim"][:2]) == [2, 3]
    assert i2["n_hit"] == 1 and list(i2["victim"][:1]) == [0] and list(i2["evicted"][:1]) == [1]
    assert list(i3["victim"][:2]) == [2, 3] and list(i3["evicted"][:2]) == [3, 4]
    # after step 3: slot0 pos5 last2, slot1 pos2 last2, slot2 pos6 last3, slot3 pos7 last3
    # step 4: 6 hits slot 2; 1 misses; candidates slots 0,1,3 -> (2,0) is smallest
    assert i4["n_hit"] == 1 and list(i4["victim"][:1]) == [0] and list(i4["evicted"][:1]) == [5]


@pytest.mark.parametrize("seed", range(6))
def test_inclusion_between_two_capacities(seed):
    rng = np.random.default_rng(200 + seed)
    h, k = 80, 6
    rows = rows_for(h)
    small, big = oracle.Cache(2 * k, h), oracle.Cache(5 * k, h)
    used_at = np.full(h, -1)
    for t, sel in enumerate(random_stream(rng, h, k, 40, 0.5)):
        small.step(t, sel, rows)
        big.step(t, sel, rows)
        used_at[sel] = t
        rs = small.pos_of()
        rs = rs[rs >= 0]
        rb = set(big.pos_of()[big.pos_of() >= 0].tolist())
        tstar = used_at[rs].min()
        # positions the small cache holds from after its boundary step are in
        # the big one; at the boundary step slot order may break ties apart
        assert all(p in rb for p in rs if used_at[p] > tstar)


def test_rejects_bad_selection():
    rows = rows_for(10)
    c = oracle.Cache(4, 10)
    with pytest.raises(ValueError):
        c.step(0, np.array([1, 2, 3, 4, 5], np.int32), rows)   # K > C
    with pytest.raises(ValueError):
        c.step(0, np.array([10], np.int32), rows)              # position >= hcap
