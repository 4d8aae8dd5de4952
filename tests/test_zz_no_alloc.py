"""The attention entry point that allocates nothing (hc_attend_cached_noalloc)
against hc_attend_cached, through the C ABI.

For callers that cannot allocate device memory: the split partials live in a
scratch array the library holds per GPU instead of a caller-owned buffer.
The kernels are the same, so the outputs must agree bit for bit.  Two calls
in a row, the second with a smaller input (fewer heads, then another context
with fewer layers), so that what the first call left in the shared scratch
cannot leak into the second; a request beyond the array's size is refused.
"""
import math

import numpy as np
import pytest

from cache_gather_amd import workload as W

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(576.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from cache_gather_amd import hc
    hc.lib()
    assert "libhc.so" in open("/proc/self/maps").read()
    yield


def _both(p, t, heads):
    """(attend_cached output, attend_cached_noalloc output) after step t."""
    import torch
    q = torch.from_numpy(W.queries(p.wl, t, heads, p.Q).view(np.int16)).cuda()
    work, ref = p.hc.attention_buffers(heads)
    out = torch.full_like(ref, float("nan"))
    p.hc.attend_cached(q, heads, SCALE, work, ref)
    p.hc.attend_cached_noalloc(q, heads, SCALE, out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def _same(a, b, msg):
    assert a.shape == b.shape, msg
    bad = np.flatnonzero(a.view(np.uint32).ravel() != b.view(np.uint32).ravel())
    assert bad.size == 0, "%s: %d values differ, first at flat index %d" % (msg, bad.size, bad[0])


def test_noalloc_matches_attend_cached_two_calls_second_smaller():
    from gpu_harness import Pair, say
    wl = W.TINY.with_(name="noalloc_a", n_sessions=2, n_layers=3, layers_per_select=2,
                      sigma_bias=(0.5, 0.5), sigma_noise=(1.0, 1.0), top_k=1000,
                      cache_slots=2048, steps=2)
    p = Pair(wl)
    p.fill_only = True          # rows straight from the slots, no bf16 buffer
    for t in range(2):
        g, o = p.step(t)
        p.compare(t, g, o)
    ref, got = _both(p, 1, 192)                  # first call: 3 head groups
    _same(ref, got, "192 heads")
    ref, got = _both(p, 1, 64)                   # second call, smaller: 1 head group
    _same(ref, got, "64 heads after 192")
    p.close()
    # a second context with a smaller shape reuses the same scratch
    p = Pair(W.TINY.with_(name="noalloc_b", steps=2))
    p.fill_only = True
    for t in range(2):
        g, o = p.step(t)
        p.compare(t, g, o)
    ref, got = _both(p, 1, 64)
    _same(ref, got, "second context")
    say("noalloc: bit-identical to attend_cached on three calls")
    p.close()


def test_noalloc_refuses_beyond_its_scratch():
    """8 layers x 4,096 heads needs more partials than the scratch holds:
    HC_E_NOMEM, nothing launched; a call that fits still matches."""
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(name="noalloc_big", n_layers=8, layers_per_select=4, steps=1))
    g, o = p.step(0)
    p.compare(0, g, o)
    heads = 4096
    assert hc.hc_attend_workspace_bytes(p.hc.ctx, heads) > hc.ATTEND_STATIC_BYTES
    q = torch.zeros((1, 8, heads, 576), dtype=torch.int16, device="cuda")
    out = torch.empty((1, 8, heads, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(hc.HcError) as e:
        p.hc.attend_cached_noalloc(q, heads, SCALE, out)
    assert e.value.status == -2
    ref, got = _both(p, 0, 64)
    _same(ref, got, "after a refused call")
    p.close()
