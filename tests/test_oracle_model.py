"""Pins of the oracle's whole decode step (selection groups, layers, gather)
and of the seeded workload generator.

Some layers reuse the selection of an earlier layer while keeping their own KV
rows (page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "Separate historical capacity from the current working set").  With a
shared selection and cold caches, every layer of a group sees the same slot
maps; the gather must return, for each selected position, the dequantised
host row (resident bytes equal host bytes).
"""
import numpy as np
import pytest

import oracle
from cache_gather_amd import workload as W


def _model(wl, n_rows=None):
    rows = [[W.fill_rows(wl, s, l) for l in range(wl.n_layers)] for s in range(wl.n_sessions)]
    m = oracle.Model(wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k,
                     wl.cache_slots, wl.hcap, rows)
    return m, rows


SMALL = W.Workload("small_groups", 2, 5, 2, 700, 12, 96, 48, (0.5, 0.2), (1.0, 1.0), 77)


def test_groups_share_selection_and_slot_maps_and_gather_is_host_dequant():
    wl = SMALL
    m, rows = _model(wl)
    sc = W.Scores(wl)
    for t in range(wl.steps):
        scores = sc.step(t)
        sel, out, infos = m.step(t, list(scores), wl.hist_len(t).astype(np.int64))
        for s in range(wl.n_sessions):
            for g in range(wl.n_groups):
                u = s * wl.n_groups + g
                np.testing.assert_array_equal(sel[s, g], oracle.topk(scores[u][:wl.hist0 + t],
                                                                     wl.top_k))
                layers = range(g * wl.layers_per_select,
                               min((g + 1) * wl.layers_per_select, wl.n_layers))
                first = None
                for l in layers:
                    info = infos[s * wl.n_layers + l]
                    if first is None:
                        first = info
                    for key in ("slot", "miss_pos", "victim", "evicted"):
                        np.testing.assert_array_equal(info[key], first[key])
                    want = np.stack([oracle.dequant_row(rows[s][l][p]) for p in sel[s, g]])
                    np.testing.assert_array_equal(out[s, l], want)
    m.close()


def test_threads_do_not_change_results():
    wl = SMALL
    m1, _ = _model(wl)
    m4, _ = _model(wl)
    sc = W.Scores(wl)
    for t in range(6):
        scores = list(sc.step(t))
        hl = wl.hist_len(t).astype(np.int64)
        a = m1.step(t, scores, hl, nthreads=1)
        b = m4.step(t, scores, hl, nthreads=4)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_tiny_workload_statistics_are_sane():
    wl = W.TINY
    m, _ = _model(wl)
    sc = W.Scores(wl)
    misses, evictions = [], 0
    for t in range(wl.steps):
        _, _, infos = m.step(t, list(sc.step(t)), wl.hist_len(t).astype(np.int64),
                             gather=False)
        misses.append(infos[0]["n_miss"])
        evictions += infos[0]["n_evict"]
    assert misses[0] == wl.top_k                 # cold cache
    assert all(0 <= x <= wl.top_k for x in misses)
    # union of 16 selections of 256 from 4,096 exceeds 1,024 slots: evictions occur
    assert evictions > 0
    m.close()


def test_generator_is_seeded_and_shaped():
    wl = W.TINY
    a = W.fill_rows(wl, 0, 0, n_rows=1000)
    b = W.fill_rows(wl, 0, 0, n_rows=1000)
    np.testing.assert_array_equal(a, b)
    q = a[:, :512].view(np.int8)
    assert q.min() == -127 and q.max() == 127
    sc = a[:, 512:528].copy().view(np.float16).astype(np.float32)
    assert sc.min() >= 1e-3 * 0.999 and sc.max() <= 0.1 * 1.001
    rope = a[:, 528:656].copy().view(np.uint16)
    # bf16 of N(0,1): exponents in a sane range, both signs present
    assert (rope >> 15).mean() == pytest.approx(0.5, abs=0.05)
    # rows of another layer differ
    c = W.fill_rows(wl, 0, 1, n_rows=1000) if wl.n_layers > 1 else W.fill_rows(
        wl.with_(n_layers=2), 0, 1, n_rows=1000)
    assert not np.array_equal(a, c)
    s1 = W.Scores(wl).unit(0, 0, 3)
    s2 = W.Scores(wl).unit(0, 0, 3)
    np.testing.assert_array_equal(s1, s2)
    assert s1.size == wl.hist0 + 3 and s1.dtype == np.float32
