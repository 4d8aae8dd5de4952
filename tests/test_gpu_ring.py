"""GPU parity of the recent ring, the batched copyback and the flush boundary.

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading": new
KV enters a GPU recent ring and reaches RAM history through a batched
copyback (data-flow figure of "Decision three"; 64-row batches in "Decision
two"); the ring protects rows not yet in RAM ("GPU cache management has
hazards too"); before history is exported, the remaining rows are submitted,
the copy is waited for and the host row count must match the logical count
("Capacity optimization must survive the session lifecycle").

Every comparison is bit-exact against the oracle, which models the ring and
its copybacks with its own host row store: selections, traces (ring rows
counted and named C + p % ring_rows), outputs, slot maps, and the pinned host
rows after every step (copied rows equal, rows not copied yet untouched).
"""
import numpy as np
import pytest

from cache_gather_amd import workload as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from cache_gather_amd import hc
    hc.lib()
    assert "libhc.so" in open("/proc/self/maps").read()
    yield


def _pair(wl, ring, batch, **kw):
    from gpu_harness import RingPair
    return RingPair(wl, ring, batch, **kw)


@pytest.mark.parametrize("ring,batch", [(8, 4), (16, 16), (8, 1), (64, 8)])
def test_ring_tiny(ring, batch):
    p = _pair(W.TINY, ring, batch)
    p.run()
    p.close()


def test_ring_sessions_layers_and_skipped_appends():
    wl = W.TINY.with_(name="tiny_ring_3x3", n_sessions=3, n_layers=3, layers_per_select=2,
                      steps=24, sigma_bias=(0.5, 1.0, 0.2), sigma_noise=(1.0, 0.3, 1.0))
    p = _pair(wl, 16, 8, skip=lambda t, s: s == 1 and t % 3 == 0)
    p.run()
    assert p.end[0] == p.first + 24 and p.end[1] == p.first + 24 - 8
    p.close()


def test_flush_midway_then_continue():
    from gpu_harness import say
    p = _pair(W.TINY.with_(steps=20), 16, 8)
    for t in range(11):
        g, o = p.step(t)
        p.compare(t, g, o)
    status, counts, o_counts = p.flush_both()
    assert status == 0
    np.testing.assert_array_equal(counts, o_counts)
    assert counts[0] == p.first + 11
    p.compare_host()
    for t in range(11, 20):       # the next batch starts at the flushed frontier
        g, o = p.step(t)
        p.compare(t, g, o)
        p.compare_host()
    status, counts, o_counts = p.flush_both()
    assert status == 0 and counts[0] == o_counts[0] == p.first + 20
    p.compare_host()
    p.compare_state()
    say("flush midway: ok")
    p.close()


def test_ring_model78_page_batches():
    """78 layers, a selection every 4th layer, 32,768 slots, top-2,048, a ring
    of 128 rows with the page's 64-row copyback batches; 136 steps, so the
    ring wraps and appended rows that left it come back from host RAM."""
    p = _pair(W.MODEL78_50K.with_(steps=136), 128, 64)
    p.run(gather_every=8, host_every=8)
    p.close()


def test_invalid_appends_and_steps_are_rejected():
    import torch
    from cache_gather_amd import hc
    wl = W.TINY
    c = hc.HotCache(1, 2, 1, wl.cache_slots, wl.top_k, wl.hcap, 0, ring_rows=8,
                    copyback_rows=4)
    rows = torch.zeros((1, 2, 656), dtype=torch.uint8, device="cuda")
    out, sel, _ = c.alloc_outputs()
    sc = torch.zeros((2, wl.hcap), dtype=torch.float32, device="cuda")
    c.step(sc, wl.hcap, [300], out, sel)
    with pytest.raises(hc.HcError):       # below a history a step already saw
        c.append(rows, [299])
    c.append(rows, [300])
    with pytest.raises(hc.HcError):       # not the next position
        c.append(rows, [302])
    with pytest.raises(hc.HcError):       # beyond the appended rows
        c.step(sc, wl.hcap, [302], out, sel)
    with pytest.raises(hc.HcError):       # misaligned rows
        c.append(rows.view(-1)[1:657].view(1, 1, 656), [301])
    c.append(rows, [301])
    c.step(sc, wl.hcap, [302], out, sel)
    status, counts = c.flush()
    assert status == 0 and counts[0] == 302
    c.close()
    plain = hc.HotCache(1, 1, 1, wl.cache_slots, wl.top_k, wl.hcap, 0)
    with pytest.raises(hc.HcError):       # no ring configured
        plain.append(rows[:, :1], [300])
    status, counts = plain.flush()        # nothing to flush
    assert status == 0 and counts[0] == 0
    plain.close()
