"""GPU parity of multi-query (MTP verification) rounds.

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "GPU cache management has hazards too": verification processes
several query rows, and several queries can select the same missing
position; a slot filled in the round is only read in later rounds,
duplicate misses read host RAM directly, and slots used by the round are
pinned.  Each of the Q queries selects its own top-K over the same history;
the cache round runs once on the union of the Q selections.

Every comparison is bit-exact against the oracle: each query's selection,
the union trace (hits, misses, victims, evictions, ring rows), every query's
gathered rows, and the slot maps and hot rows at the end.
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


def _pair(wl, Q):
    from gpu_harness import Pair
    return Pair(wl, queries=Q)


@pytest.mark.parametrize("Q", [2, 4])
def test_tiny_rounds(Q):
    p = _pair(W.TINY, Q)
    p.run()
    p.close()


def test_eight_queries_groups_and_sessions():
    wl = W.TINY.with_(name="mtp_groups", n_sessions=2, n_layers=3, layers_per_select=2,
                      top_k=64, cache_slots=640, steps=12, sigma_bias=(0.5, 1.0),
                      sigma_noise=(1.0, 0.3))
    p = _pair(wl, 8)
    p.run()
    p.close()


def test_slots_equal_to_the_round_rows():
    """C = Q * K, the smallest cache a round is allowed: a round with Q
    disjoint selections uses every slot."""
    wl = W.TINY.with_(name="mtp_min_slots", top_k=64, cache_slots=256, steps=20,
                      sigma_bias=(0.3,), sigma_noise=(1.0,))
    p = _pair(wl, 4)
    p.run()
    assert p.evictions > 0
    p.close()


def test_identical_queries_share_every_miss():
    """All Q queries select the same positions: every miss is one fill plus
    Q - 1 rows read from host RAM, and all queries' rows are equal."""
    from gpu_harness import say
    Q = 4
    p = _pair(W.TINY.with_(steps=6), Q)
    for t in range(6):
        one = p.scores.step(t, p.stride)
        sc = np.repeat(one, Q, axis=0)
        g, o = p.step(t, scores_np=sc)
        p.compare(t, g, o)
        for q in range(1, Q):
            np.testing.assert_array_equal(g["out"][:, :, q], g["out"][:, :, 0])
        if t == 0:
            assert g["trace"][0, 1] == W.TINY.top_k   # one miss per distinct position
    p.compare_state()
    say("identical queries: ok")
    p.close()


def test_rounds_with_a_recent_ring():
    from gpu_harness import RingPair
    p = RingPair(W.TINY, 16, 8, queries=4)
    p.run()
    p.close()


def test_model78_four_query_rounds():
    """78 layers, a selection every 4th layer, 32,768 slots, top-2,048 and
    MTP = 3 (four query rows): unions of up to 8,192 positions per group."""
    p = _pair(W.MODEL78_50K, 4)
    p.run(gather_every=8)
    p.close()
