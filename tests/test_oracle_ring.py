"""Pins of the oracle's recent ring and batched copyback.

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading": in
the data-flow figure of "Decision three", new KV goes to a GPU recent ring and
reaches RAM history through a batched copyback; section "GPU cache management
has hazards too": the ring protects new rows that have not reached RAM yet;
the copyback is batched (64 rows at a time on the page, "Decision two"); and
section "Capacity optimization must survive the session lifecycle": before
history is exported, outstanding rows are submitted, the copy is waited for,
and the host row count must equal the logical count.

Readings: a ring holds the last `rows` appended rows of a (session, layer);
after an append, once `batch` appended rows are not yet in host RAM, all of
them are copied; a selected position the ring holds is read from the ring and
does not touch the LRU cache; every other selected position goes through the
LRU cache exactly as without a ring, its misses read host RAM.

Pins, none of which reuses the oracle's code:
  * the positions the ring holds, by arithmetic: first <= p and p >= end - rows;
  * the host frontier in closed form: first + floor(appended / batch) * batch,
    host bytes equal to the appended rows below it and untouched above it;
  * the cache state equals the pure-Python LRU fed only the selected positions
    the ring does not hold; the trace names ring rows C + p % rows;
  * gathered rows equal the appended rows also after they left the ring (then
    they come from host RAM, so a lost copyback would show);
  * flush moves the frontier to the end and the host bytes follow.
"""
import numpy as np
import pytest

import oracle
from test_oracle_lru import PyLRU


def _frontier(first, end, batch):
    return first + (end - first) // batch * batch


def _in_ring(p, first, end, rows):
    return first <= p < end and p >= end - rows


def _scores(rng, h, first):
    # recent positions score higher on average, so the ring is selected from
    s = rng.standard_normal(h).astype(np.float32)
    s[first:] += np.float32(1.5)
    return s


@pytest.mark.parametrize("rows,batch", [(16, 4), (16, 16), (8, 1), (128, 64)])
def test_ring_step_by_step(rows, batch):
    first, hcap, K, C, steps = 200, 300, 24, 48, 80
    rng = np.random.default_rng(rows * 100 + batch)
    all_rows = rng.integers(0, 256, (hcap, 656), dtype=np.uint8)
    host = np.zeros((hcap, 656), np.uint8)
    host[:first] = all_rows[:first]
    m = oracle.Model(1, 1, 1, K, C, hcap, [[host]], ring_rows=rows, copyback_rows=batch)
    ref = PyLRU(C)
    for t in range(steps):
        p_new = first + t
        m.append([p_new], [[all_rows[p_new]]])
        end = p_new + 1
        fr = _frontier(first, end, batch)
        assert m.ring(0, 0).copied() == fr
        np.testing.assert_array_equal(host[first:fr], all_rows[first:fr])
        assert not host[fr:].any()
        sc = _scores(rng, end, first)
        sel, out, infos = m.step(t, [sc], [end])
        sel = sel[0, 0]
        np.testing.assert_array_equal(sel, oracle.topk(sc, K))
        info = infos[0]
        ring_mask = np.array([_in_ring(p, first, end, rows) for p in sel])
        assert info["n_ring"] == ring_mask.sum()
        assert info["n_hit"] + info["n_miss"] + info["n_ring"] == K
        for p in sel[ring_mask]:
            assert m.ring(0, 0).holds(p)
        events = ref.step(t, [int(p) for p in sel[~ring_mask]])
        assert info["n_miss"] == len(events)
        np.testing.assert_array_equal(info["miss_pos"][:len(events)], [e[0] for e in events])
        np.testing.assert_array_equal(info["victim"][:len(events)], [e[1] for e in events])
        np.testing.assert_array_equal(info["evicted"][:len(events)], [e[2] for e in events])
        want_slot = [C + int(p) % rows if r else ref.slot_of(int(p)) for p, r in zip(sel, ring_mask)]
        np.testing.assert_array_equal(info["slot"], want_slot)
        # ring rows never enter the cache
        slot_of = m.cache(0, 0).slot_of()
        for p in sel[ring_mask]:
            if ref.slot_of(int(p)) < 0:
                assert slot_of[p] == -1
        # every gathered row is the dequantised appended / prefill row
        for i in rng.choice(K, 6, replace=False):
            np.testing.assert_array_equal(out[0, 0, i], oracle.dequant_row(all_rows[sel[i]]))
    end = first + steps
    assert m.flush() == [end]
    np.testing.assert_array_equal(host[first:end], all_rows[first:end])
    assert not host[end:].any()
    m.close()


def test_rows_that_left_the_ring_come_from_host_ram():
    """A position selected after it left the ring misses and is fetched from
    host RAM, where only the copyback can have put it."""
    first, hcap, K, C, rows, batch = 64, 128, 8, 16, 8, 4
    rng = np.random.default_rng(3)
    all_rows = rng.integers(0, 256, (hcap, 656), dtype=np.uint8)
    host = np.zeros((hcap, 656), np.uint8)
    host[:first] = all_rows[:first]
    m = oracle.Model(1, 1, 1, K, C, hcap, [[host]], ring_rows=rows, copyback_rows=batch)
    target = first + 2
    for t in range(20):
        m.append([first + t], [[all_rows[first + t]]])
        end = first + t + 1
        sc = np.full(end, -1.0, np.float32)
        sc[:K] = 0.0                  # K - 1 old positions and the target win
        sc[K - 1] = -2.0
        if target < end:
            sc[target] = 5.0
        sel, out, infos = m.step(t, [sc], [end])
        if t >= 2:
            i = int(np.flatnonzero(sel[0, 0] == target)[0])
            np.testing.assert_array_equal(out[0, 0, i], oracle.dequant_row(all_rows[target]))
            in_ring = _in_ring(target, first, end, rows)
            assert m.ring(0, 0).holds(target) == in_ring
            if not in_ring and m.cache(0, 0).slot_of()[target] >= 0:
                hot = m.cache(0, 0).hot()[m.cache(0, 0).slot_of()[target]]
                np.testing.assert_array_equal(hot, all_rows[target])
    # the target left the ring at end = target + rows + 1 and was then fetched
    assert m.cache(0, 0).slot_of()[target] >= 0
    m.close()


def test_several_sessions_layers_and_skipped_appends():
    S, L, R, K, C, rows, batch = 2, 3, 2, 16, 32, 8, 4
    first, hcap, steps = [100, 120], 200, 30
    rng = np.random.default_rng(11)
    all_rows = [[rng.integers(0, 256, (hcap, 656), dtype=np.uint8) for _ in range(L)]
                for _ in range(S)]
    host = [[np.zeros((hcap, 656), np.uint8) for _ in range(L)] for _ in range(S)]
    for s in range(S):
        for l in range(L):
            host[s][l][:first[s]] = all_rows[s][l][:first[s]]
    m = oracle.Model(S, L, R, K, C, hcap, host, ring_rows=rows, copyback_rows=batch)
    end = list(first)
    G = (L + R - 1) // R
    for t in range(steps):
        pos = [end[0], end[1] if t % 2 == 0 else None]   # session 1 appends every other step
        m.append(pos, [[all_rows[s][l][end[s]] for l in range(L)] for s in range(S)])
        for s in range(S):
            if pos[s] is not None:
                end[s] += 1
        scores = [_scores(rng, end[u // G], first[u // G]) for u in range(S * G)]
        sel, out, infos = m.step(t, scores, end)
        for s in range(S):
            fr = _frontier(first[s], end[s], batch)
            for l in range(L):
                assert m.ring(s, l).copied() == fr
                np.testing.assert_array_equal(host[s][l][first[s]:fr], all_rows[s][l][first[s]:fr])
                assert not host[s][l][fr:].any()
                info = infos[s * L + l]
                sv = sel[s, l // R]
                n_ring = sum(_in_ring(p, first[s], end[s], rows) for p in sv)
                assert info["n_ring"] == n_ring
                i = int(rng.integers(K))
                np.testing.assert_array_equal(out[s, l, i], oracle.dequant_row(all_rows[s][l][sv[i]]))
    assert m.flush() == end
    m.close()


def test_out_of_order_appends_are_rejected():
    r = oracle.Ring(8, 4)
    host = np.zeros((64, 656), np.uint8)
    row = np.ones(656, np.uint8)
    r.append(10, row, host)
    with pytest.raises(ValueError):
        r.append(12, row, host)
    with pytest.raises(ValueError):
        r.append(10, row, host)
    r.append(11, row, host)
    assert r.copied() == 10 and not host.any()
    assert r.flush(host) == 12
    assert host[10:12].all() and not host[:10].any() and not host[12:].any()
    with pytest.raises(ValueError):
        oracle.Ring(4, 8)          # a batch larger than the ring
    r.close()


def test_flush_before_any_append_reports_zero():
    r = oracle.Ring(8, 4)
    host = np.zeros((16, 656), np.uint8)
    assert r.flush(host) == 0 and not r.holds(0)
    r.close()
