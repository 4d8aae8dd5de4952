"""Pins of the oracle's multi-query round (MTP verification).

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "GPU cache management has hazards too": verification processes
several query rows, and several queries can select the same missing
position; slots used by the current round are pinned; a slot filled in the
round is only a hit source in the next round, and duplicate misses read host
RAM directly.  Reading: each of the Q queries selects its own top-K over the
same history; the cache step runs once on the ascending union of the Q
selections (a position selected by several queries is one hit, or one miss
with one victim); each query's rows are gathered in its own selection order.

Pins, none of which reuses the oracle's code:
  * each query's selection equals a numpy lexsort top-K on IEEE totalOrder keys;
  * the union is numpy's union1d; the cache state and the miss / victim /
    eviction lists equal the pure-Python LRU stepped on that union;
  * every gathered row equals the dequantised host row of its position;
  * closed forms: Q identical queries give one selection's worth of misses;
    Q disjoint selections fill Q*K slots; Q = 1 gives the single-query step.
"""
import numpy as np
import pytest

import oracle
from test_oracle_lru import PyLRU


def _ref_topk(x, k):
    b = x.astype(np.float32).view(np.uint32).astype(np.int64)
    key = np.where(b & 0x80000000, 0xFFFFFFFF - b, b | 0x80000000)
    order = np.lexsort((np.arange(x.size), -key))
    return np.sort(order[:k]).astype(np.int32)


def _rows(h, seed):
    return np.random.default_rng(seed).integers(0, 256, (h, 656), dtype=np.uint8)


@pytest.mark.parametrize("Q,locality", [(4, 0.9), (4, 0.3), (2, 0.6), (8, 0.8)])
def test_union_round_against_python_lru(Q, locality):
    H, K, C, steps = 3000, 64, 512, 12
    rng = np.random.default_rng(Q * 10 + int(locality * 10))
    rows = _rows(H, 5)
    m = oracle.Model(1, 1, 1, K, C, H, [[rows]], queries=Q)
    ref = PyLRU(C)
    base = rng.standard_normal(H).astype(np.float32)
    for t in range(steps):
        # queries share a base score (overlapping selections) plus their own noise
        sc = [(np.float32(locality) * base + np.float32(1 - locality) *
               rng.standard_normal(H).astype(np.float32)) for _ in range(Q)]
        sel, out, infos = m.step(t, sc, [H])
        assert sel.shape == (1, 1, Q, K) and out.shape == (1, 1, Q, K, 576)
        for q in range(Q):
            np.testing.assert_array_equal(sel[0, 0, q], _ref_topk(sc[q], K))
        union = np.union1d(np.concatenate([sel[0, 0, q] for q in range(Q)]), [])
        union = union.astype(np.int64)
        info = infos[0]
        n = union.size
        assert info["n_hit"] + info["n_miss"] + info["n_ring"] == n and info["n_ring"] == 0
        events = ref.step(t, [int(p) for p in union])
        assert info["n_miss"] == len(events)
        np.testing.assert_array_equal(info["miss_pos"][:len(events)], [e[0] for e in events])
        np.testing.assert_array_equal(info["victim"][:len(events)], [e[1] for e in events])
        np.testing.assert_array_equal(info["evicted"][:len(events)], [e[2] for e in events])
        np.testing.assert_array_equal(info["slot"][:n], [ref.slot_of(int(p)) for p in union])
        assert np.all(info["slot"][n:] == -1) and np.all(info["miss_pos"][len(events):] == -1)
        for q in range(Q):
            for i in rng.choice(K, 4, replace=False):
                np.testing.assert_array_equal(out[0, 0, q, i],
                                              oracle.dequant_row(rows[sel[0, 0, q, i]]))
    m.close()


def test_identical_queries_miss_once():
    H, K, C, Q = 2000, 128, 512, 4
    rows = _rows(H, 7)
    m = oracle.Model(1, 1, 1, K, C, H, [[rows]], queries=Q)
    x = np.random.default_rng(1).standard_normal(H).astype(np.float32)
    sel, out, infos = m.step(0, [x] * Q, [H])
    assert infos[0]["n_miss"] == K and infos[0]["n_hit"] == 0
    np.testing.assert_array_equal(infos[0]["victim"][:K], np.arange(K))
    for q in range(1, Q):
        np.testing.assert_array_equal(sel[0, 0, q], sel[0, 0, 0])
        np.testing.assert_array_equal(out[0, 0, q], out[0, 0, 0])
    sel, out, infos = m.step(1, [x] * Q, [H])
    assert infos[0]["n_miss"] == 0 and infos[0]["n_hit"] == K
    m.close()


def test_disjoint_queries_fill_q_times_k_slots():
    H, K, Q = 4096, 100, 4
    C = Q * K
    rows = _rows(H, 9)
    m = oracle.Model(1, 1, 1, K, C, H, [[rows]], queries=Q)
    sc = []
    for q in range(Q):
        x = np.zeros(H, np.float32)
        x[q * 1000:q * 1000 + K] = 1.0       # query q selects [1000q, 1000q + K)
        sc.append(x)
    sel, out, infos = m.step(0, sc, [H])
    info = infos[0]
    assert info["n_miss"] == Q * K
    want = np.concatenate([np.arange(q * 1000, q * 1000 + K) for q in range(Q)])
    np.testing.assert_array_equal(info["miss_pos"], want)
    np.testing.assert_array_equal(info["victim"], np.arange(Q * K))
    assert (m.cache(0, 0).pos_of() >= 0).all()
    m.close()


def test_one_query_is_the_single_query_step():
    H, K, C = 3000, 64, 256
    rows = _rows(H, 11)
    a = oracle.Model(1, 2, 1, K, C, H, [[rows, rows]])
    b = oracle.Model(1, 2, 1, K, C, H, [[rows, rows]], queries=1)
    rng = np.random.default_rng(2)
    for t in range(6):
        sc = [rng.standard_normal(H).astype(np.float32) for _ in range(2)]
        ra, rb = a.step(t, sc, [H]), b.step(t, sc, [H])
        np.testing.assert_array_equal(ra[0], rb[0])
        np.testing.assert_array_equal(ra[1], rb[1])
    a.close()
    b.close()


def test_ring_rows_leave_the_union_cache_step():
    """With a recent ring, union positions the ring holds skip the cache."""
    H0, K, C, Q, rows_ring = 500, 32, 256, 4, 16
    hcap = H0 + 20
    allr = _rows(hcap, 13)
    host = np.zeros_like(allr)
    host[:H0] = allr[:H0]
    m = oracle.Model(1, 1, 1, K, C, hcap, [[host]], ring_rows=rows_ring, copyback_rows=8,
                     queries=Q)
    rng = np.random.default_rng(4)
    for t in range(20):
        m.append([H0 + t], [[allr[H0 + t]]])
        end = H0 + t + 1
        sc = []
        for q in range(Q):
            x = rng.standard_normal(end).astype(np.float32)
            x[H0:] += 2.0
            sc.append(x)
        sel, out, infos = m.step(t, sc, [end])
        union = np.union1d(np.concatenate([sel[0, 0, q] for q in range(Q)]), [])
        in_ring = (union >= H0) & (union >= end - rows_ring)
        assert infos[0]["n_ring"] == in_ring.sum()
        assert infos[0]["n_hit"] + infos[0]["n_miss"] + infos[0]["n_ring"] == union.size
        for q in range(Q):
            i = int(rng.integers(K))
            np.testing.assert_array_equal(out[0, 0, q, i], oracle.dequant_row(allr[sel[0, 0, q, i]]))
    m.close()
