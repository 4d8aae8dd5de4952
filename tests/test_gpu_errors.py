"""The C ABI's failure paths on the GPU.

Page "Making KV offload correct" (richardcheam.github.io): sections "A grouped
allocation is a transaction" (hc_create is all-or-nothing), "Response
completion is not copy completion" (hc_destroy waits for queued work) and
"What I tested and what each check could show" (failures must surface, not
pass silently).  Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
Offloading", section "GPU cache management has hazards too" (a slot filled in
a round is not read before its fill).

* A rejected hc_step (each argument check) returns HC_E_INVAL and changes
  nothing: the run continues bit-exact with the oracle.
* With the test build libhc_test.so (include/hc_test.h), every failure is
  forced from the host while every kernel keeps its indexes in range: a launch
  failure gives HC_E_HIP and then HC_E_STATE on every call but hc_destroy; a
  select kernel that finds its scan state inconsistent, and an LRU queue too
  short for the step's misses, give HC_E_DEVICE at the next check and then
  HC_E_STATE; a pinned host allocation failing inside hc_create leaves no
  pinned memory behind; and victim slots overwritten with a sentinel before
  each gather leave every output bit-exact (no read before the fill).
* hc_destroy with steps still queued, steps alternating between two streams,
  and hc_attend_cached after an hc_append (refused: the ring may no longer
  hold the step's rows).
"""
import math

import numpy as np
import pytest

from cache_gather_amd import workload as W

pytestmark = pytest.mark.gpu

E_INVAL, E_NOMEM, E_HIP, E_STATE, E_DEVICE = -1, -2, -3, -4, -6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from cache_gather_amd import hc
    hc.lib()
    hc.test_lib()
    maps = open("/proc/self/maps").read()
    assert "libhc.so" in maps and "libhc_test.so" in maps
    yield


def _status(fn, *args):
    from cache_gather_amd import hc
    try:
        fn(*args)
    except hc.HcError as e:
        return e.status
    return 0


def test_rejected_steps_change_nothing():
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(steps=8))
    for t in range(3):
        g, o = p.step(t)
        p.compare(t, g, o)
    wl, ctx = p.wl, p.hc.ctx
    st = torch.cuda.current_stream().cuda_stream
    p.d_scores.copy_(torch.from_numpy(p.scores_for(3)))
    h = int(wl.hist_len(3)[0])

    def step(hist, stride=p.stride, scores=p.d_scores, out=p.out, sel=p.sel):
        return _status(hc.hc_step, ctx, st, scores, stride, [hist], out, sel, p.trace)

    assert step(int(wl.hist_len(1)[0])) == E_INVAL          # history shorter than last step's
    assert step(wl.top_k - 1) == E_INVAL                    # fewer positions than K
    assert step(wl.hcap + 1) == E_INVAL                     # beyond the host rows
    assert step(h, stride=h - 1) == E_INVAL                 # score rows shorter than the history
    assert step(h, out=p.out.view(-1)[1:]) == E_INVAL       # output not 16-byte aligned
    assert step(h, scores=None) == E_INVAL
    assert step(h, sel=None) == E_INVAL
    assert hc.hc_steps_done(ctx) == 3
    for t in range(3, 8):
        g, o = p.step(t)
        p.compare(t, g, o)
    p.compare_state()
    p.close()


def test_launch_failure_poisons_the_context():
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    with hc.using(hc.test_lib()):
        p = Pair(W.TINY.with_(steps=3))
        g, o = p.step(0)
        p.compare(0, g, o)
        ctx = p.hc.ctx
        st = torch.cuda.current_stream().cuda_stream
        hc.hc_test_hook(ctx, hc.TEST_FAIL_LAUNCH)
        p.d_scores.copy_(torch.from_numpy(p.scores_for(1)))
        args = (ctx, st, p.d_scores, p.stride, p.wl.hist_len(1), p.out, p.sel, p.trace)
        assert _status(hc.hc_step, *args) == E_HIP
        assert hc.hc_steps_done(ctx) == 1                   # the failed step did not count
        assert _status(hc.hc_step, *args) == E_STATE
        assert _status(hc.hc_export_state, ctx, 0, 0, p.wl.cache_slots, p.wl.hcap) == E_STATE
        assert hc.hc_flush(ctx, st, 1, check=False)[0] == E_STATE
        assert _status(hc.hc_profile_enable, ctx, 1) == E_STATE
        work, out = p.hc.attention_buffers(64)
        q = torch.zeros((1, 1, 64, 576), dtype=torch.int16, device="cuda")
        assert _status(hc.hc_attend_cached, ctx, st, q, 64, 0.1, work, work.numel(), out) == E_STATE
        p.close()                                           # hc_destroy still works


@pytest.mark.parametrize("queries", [1, 2])
def test_select_inconsistency_is_reported(queries):
    """The select kernels' guard (its scan state does not add up) reports
    through the context's error words: HC_E_DEVICE at the next check, then
    HC_E_STATE.  With two query rows the round kernel's guard reports too."""
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    with hc.using(hc.test_lib()):
        for first_check in ("step", "export"):
            p = Pair(W.TINY.with_(steps=4), queries=queries)
            for t in range(2):
                g, o = p.step(t)
                p.compare(t, g, o)
            hc.hc_test_hook(p.hc.ctx, hc.TEST_FORCE_SELECT)
            p.gpu_step(2, p.scores_for(2), p.wl.hist_len(2))   # enqueued: HC_OK
            torch.cuda.synchronize()
            if first_check == "step":
                assert _status(p.gpu_step, 3, p.scores_for(3), p.wl.hist_len(3)) == E_DEVICE
            else:
                assert _status(p.hc.export_state, 0, 0) == E_DEVICE
            assert _status(p.gpu_step, 3, p.scores_for(3), p.wl.hist_len(3)) == E_STATE
            assert _status(p.hc.export_state, 0, 0) == E_STATE
            p.close()


def test_lru_queue_corruption_is_reported():
    """A unit whose LRU claims every slot used but whose queue is empty cannot
    find victims for its misses: the select kernel reports it (HC_E_DEVICE
    from hc_flush, then HC_E_STATE)."""
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    with hc.using(hc.test_lib()):
        p = Pair(W.TINY.with_(steps=4))
        for t in range(2):
            g, o = p.step(t)
            p.compare(t, g, o)
        hc.hc_test_hook(p.hc.ctx, hc.TEST_CORRUPT_LRU)
        p.gpu_step(2, p.scores_for(2), p.wl.hist_len(2))
        torch.cuda.synchronize()
        assert int(p.trace[0, 1].item()) > 0                # the step had misses to place
        assert _status(p.hc.flush) == E_DEVICE
        assert _status(p.hc.flush) == E_STATE
        p.close()


def test_failed_create_leaves_no_pinned_memory():
    import torch
    from cache_gather_amd import hc
    with hc.using(hc.test_lib()):
        before = hc.hc_test_hook(None, hc.TEST_PINNED_BYTES)
        cfg = hc.make_config(2, 3, 2, 600, 256, 5000, ring_rows=8, copyback_rows=4)
        n = hc.hc_workspace_bytes(cfg)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        # the 6 row stores, the ring's host counts, the error words: fail each in turn
        for k in range(8):
            hc.hc_test_hook(None, hc.TEST_FAIL_PINNED, k)
            assert _status(hc.hc_create, cfg, ws, n) == E_NOMEM, k
            assert hc.hc_test_hook(None, hc.TEST_PINNED_BYTES) == before, k
        hc.hc_test_hook(None, hc.TEST_FAIL_PINNED, -1)
        assert _status(hc.hc_create, cfg, ws, n - 1) == E_NOMEM       # workspace too small
        bad = hc.make_config(2, 3, 2, 600, 256, 5000, device=4096)
        assert _status(hc.hc_create, bad, ws, n) == E_INVAL           # no such device
        assert hc.hc_test_hook(None, hc.TEST_PINNED_BYTES) == before
        ctx = hc.hc_create(cfg, ws, n)
        held = hc.hc_test_hook(None, hc.TEST_PINNED_BYTES) - before
        assert held == 6 * 5000 * 656 + 2 * 8 + 4 * 4
        hc.hc_destroy(ctx)
        assert hc.hc_test_hook(None, hc.TEST_PINNED_BYTES) == before


@pytest.mark.parametrize("queries", [1, 2])
def test_victim_slots_are_not_read_before_their_fill(queries):
    """Every victim slot of every layer holds a sentinel when the gather
    starts; outputs stay bit-exact, so no gather workgroup reads a slot that
    the same launch fills."""
    from cache_gather_amd import hc
    from gpu_harness import Pair
    with hc.using(hc.test_lib()):
        wl = W.TINY.with_(name="poison", n_layers=3, layers_per_select=2, steps=12)
        p = Pair(wl, queries=queries)
        hc.hc_test_hook(p.hc.ctx, hc.TEST_POISON_VICTIMS, 1)
        p.run()
        assert p.evictions > 0
        p.close()


def test_destroy_with_steps_still_queued():
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    wl = W.MODEL78_50K.with_(n_layers=8, steps=8)
    c = hc.HotCache(1, 8, 4, wl.cache_slots, wl.top_k, wl.hcap, 0)
    for l in range(8):
        c.host_rows(0, l)[:] = 0
    stride = (wl.hcap + 3) // 4 * 4
    sc = W.Scores(wl)
    d = torch.empty((wl.steps, wl.n_units, stride), dtype=torch.float32, device="cuda")
    for t in range(wl.steps):
        d[t].copy_(torch.from_numpy(sc.step(t, stride)))
    torch.cuda.synchronize()
    out, sel, _ = c.alloc_outputs()
    for t in range(wl.steps):
        c.step(d[t], stride, wl.hist_len(t), out, sel)
    c.close()                                  # waits for the queued steps, then frees
    torch.cuda.synchronize()
    p = Pair(W.TINY.with_(steps=2))            # the device is still fine
    for t in range(2):
        g, o = p.step(t)
        p.compare(t, g, o)
    p.close()


def test_steps_on_two_streams_are_ordered():
    """Consecutive steps on two streams, all enqueued before any wait, with
    no synchronisation by the caller: the library orders each call after the
    context's earlier work, and every step stays bit-exact."""
    import torch
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(steps=8))
    wl, steps = p.wl, 8
    scores = [p.scores_for(t) for t in range(steps)]
    d_scores = [torch.from_numpy(x).cuda() for x in scores]
    outs = [p.hc.alloc_outputs(trace=True) for _ in range(steps)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for t in range(steps):
        out, sel, tr = outs[t]
        p.hc.step(d_scores[t], p.stride, wl.hist_len(t), out, sel, tr, stream=streams[t % 2])
    for t in range(steps):
        o = p.orc.step(t, list(scores[t]), np.asarray(wl.hist_len(t), np.int64))
        if t == 0:
            torch.cuda.synchronize()
        out, sel, tr = outs[t]
        g = {"sel": sel.cpu().numpy(), "trace": tr.cpu().numpy(),
             "out": out.cpu().numpy().view(np.uint16)}
        p.compare(t, g, o)
    p.compare_state()
    p.close()


def test_attend_cached_after_an_append_is_refused():
    import torch
    from cache_gather_amd import hc
    from gpu_harness import RingPair
    p = RingPair(W.TINY.with_(steps=4), 16, 8, recent_boost=2.0)
    heads, scale = 64, 1.0 / math.sqrt(576.0)
    work, out = p.hc.attention_buffers(heads)
    q = torch.from_numpy(W.queries(p.wl, 0, heads, 1).view(np.int16)).cuda()
    g, o = p.step(0)
    p.compare(0, g, o)
    p.hc.attend_cached(q, heads, scale, work, out)           # allowed right after a step
    p.d_new.zero_()
    p.hc.append(p.d_new, [p.end[0]])
    p.orc.append([p.end[0]], np.zeros((1, 1, 656), np.uint8))
    p.end[0] += 1
    st = torch.cuda.current_stream().cuda_stream
    assert _status(hc.hc_attend_cached, p.hc.ctx, st, q, heads, scale, work, work.numel(),
                   out) == E_INVAL
    p.hc.attend(q, heads, scale, p.out, work, out)            # the buffer path is unaffected
    torch.cuda.synchronize()
    p.close()
