"""GPU parity over seeded random configurations.

The draws (tests/sweep_cases.py) mix sessions, layers and ragged layer
groups, top-K from 1 to 4,096, one to four query rows, slot counts from the
round's rows to four times them, histories that differ per session and pause
on some steps, all three replacement policies, unaligned score strides and
recent rings with copyback batches.  Every step is compared bit-exact with the
oracle: selections, hit / miss / victim / eviction traces and outputs; after
the last step the slot maps and resident rows, and for ring draws the pinned
host rows and the flush.
"""
import numpy as np
import pytest

import sweep_cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from cache_gather_amd import hc
    hc.lib()
    assert "libhc.so" in open("/proc/self/maps").read()
    yield


@pytest.mark.parametrize("case", sweep_cases.CASES, ids=[c.name for c in sweep_cases.CASES])
def test_random_configuration(case):
    from gpu_harness import Pair, RingPair, align4, say
    wl = case.wl
    stride = align4(wl.hcap) + case.stride_pad
    say("sweep case", case.name, "stride", stride, "start_back", case.start_back,
        "pause", case.pause)
    if case.ring_rows:
        p = RingPair(wl, case.ring_rows, case.copyback_rows, skip=case.skip,
                     queries=case.queries, replacement=case.policy, score_stride=stride)
        p.run()
    else:
        p = Pair(wl, score_stride=stride, queries=case.queries, replacement=case.policy)
        for t in range(wl.steps):
            g, o = p.step(t, hist_len=case.hist_len(t))
            p.compare(t, g, o)
        p.compare_state()
    p.close()
