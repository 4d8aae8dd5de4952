"""GPU parity of the circular and clock replacement policies.

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "GPU cache management has hazards too": clock replacement with
reference bits was pathological on a probe with a full hot cache, all
reference bits set and 1% misses, and was replaced by circular eviction that
skips the slots pinned by the current round.  Both run here as alternatives
to LRU; the kernels take the victims by prefix counts over the circular slot
order (no sequential scan), the oracle walks the hand one slot at a time.
Every comparison is bit-exact: selections, victims and evictions, outputs,
slot maps and hot rows.
"""
import numpy as np
import pytest

from cache_gather_amd import workload as W

pytestmark = pytest.mark.gpu

CIRCULAR, CLOCK = 1, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from cache_gather_amd import hc
    hc.lib()
    assert "libhc.so" in open("/proc/self/maps").read()
    yield


def _pair(wl, policy, **kw):
    from gpu_harness import Pair
    return Pair(wl, replacement=policy, **kw)


@pytest.mark.parametrize("policy", [CIRCULAR, CLOCK])
def test_tiny_evicting(policy):
    p = _pair(W.TINY, policy)
    p.run()
    p.close()


@pytest.mark.parametrize("policy", [CIRCULAR, CLOCK])
def test_slots_not_a_multiple_of_32_and_groups(policy):
    wl = W.TINY.with_(name="odd_slots", n_sessions=2, n_layers=3, layers_per_select=2,
                      top_k=100, cache_slots=1001, steps=30, sigma_bias=(0.3, 0.6),
                      sigma_noise=(1.0, 1.0))
    p = _pair(wl, policy)
    p.run()
    p.close()


@pytest.mark.parametrize("policy", [CIRCULAR, CLOCK])
def test_mtp_rounds(policy):
    p = _pair(W.TINY.with_(steps=12), policy, queries=4)
    p.run()
    p.close()


@pytest.mark.parametrize("policy", [CIRCULAR, CLOCK])
def test_million_position_history_evicting(policy):
    """1,048,576 positions, 32,768 slots, top-2,048, ~96% misses per step:
    eviction from step 16 on, every step bit-exact."""
    p = _pair(W.LONG_1M.with_(steps=64), policy)
    p.run(gather_every=8)
    p.close()


@pytest.mark.parametrize("policy", [CIRCULAR, CLOCK])
def test_page_probe_state(policy):
    """The page's probe: a full hot cache (32,768 slots, every reference bit
    set by the fills), then a step of 2,048 rows with 1% (20) misses."""
    from gpu_harness import say
    K, C = 2048, 32768
    wl = W.Workload("probe", 1, 1, 1, 4 * C, 17, C, K, (1.0,), (1.0,), 77)
    p = _pair(wl, policy)
    H = wl.hist0
    for t in range(C // K):               # 16 disjoint blocks fill every slot
        sc = np.zeros((1, p.stride), np.float32)
        sc[0, t * K:(t + 1) * K] = 1.0
        g, o = p.step(t, scores_np=sc, hist_len=[H], gather=False)
        p.compare(t, g, o, gather=False)
    rng = np.random.default_rng(3)
    keep = np.sort(rng.choice(C, K - 20, replace=False))
    new = np.sort(rng.choice(np.arange(C, H), 20, replace=False))
    sc = np.zeros((1, p.stride), np.float32)
    sc[0, keep] = 1.0
    sc[0, new] = 1.0
    t = C // K
    g, o = p.step(t, scores_np=sc, hist_len=[H])
    p.compare(t, g, o)
    assert g["trace"][0, 1] == 20 and g["trace"][0, 2] == 20   # 20 misses, 20 evictions
    if policy == CLOCK:
        assert o[2][0]["n_miss"] == 20
    p.compare_state()
    say("probe state, policy %d: ok" % policy)
    p.close()
