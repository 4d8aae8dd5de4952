"""The random configurations of the GPU sweep are valid and varied (CPU only):
each passes the C ABI's configuration checks, histories stay within
[top_k, hist0 + t] and never shrink, and together the draws cover every
replacement policy, rings, several query rows, unaligned strides, ragged layer
groups, paused sessions and both small and large top-K."""
import numpy as np

from cache_gather_amd import hc
import sweep_cases


def test_every_draw_is_a_valid_configuration():
    for c in sweep_cases.CASES:
        wl = c.wl
        cfg = hc.make_config(wl.n_sessions, wl.n_layers, wl.layers_per_select,
                             wl.cache_slots, wl.top_k, wl.hcap, ring_rows=c.ring_rows,
                             copyback_rows=c.copyback_rows, queries=c.queries,
                             replacement=c.policy)
        assert hc.hc_workspace_bytes(cfg) > 0, c.name


def test_histories_grow_within_bounds():
    for c in sweep_cases.CASES:
        wl = c.wl
        prev = None
        for t in range(wl.steps):
            h = c.hist_len(t).astype(np.int64)
            assert np.all(h >= wl.top_k) and np.all(h <= wl.hist0 + t), c.name
            if prev is not None:
                assert np.all(h >= prev), c.name
            prev = h
        if c.ring_rows:
            assert wl.hist0 - 1 >= wl.top_k, c.name   # a session that skips step 0


def test_draws_cover_the_options():
    cs = sweep_cases.CASES
    assert {c.policy for c in cs} == {0, 1, 2}
    assert any(c.ring_rows for c in cs) and any(not c.ring_rows for c in cs)
    assert any(c.queries > 1 for c in cs)
    assert any(c.stride_pad for c in cs)
    assert any(c.wl.n_layers % c.wl.layers_per_select for c in cs)
    assert any(max(c.pause) > 0 for c in cs)
    assert any(max(c.start_back) > 0 for c in cs)
    assert any(c.wl.n_sessions > 1 for c in cs)
    assert min(c.wl.top_k for c in cs) < 32 and max(c.wl.top_k for c in cs) >= 512
