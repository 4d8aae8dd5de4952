"""GPU parity of the attention consumer (MLA decode attention over the
selected rows) and of its fused form that never writes the bf16 buffer.

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "Decision three: let the GPU manage the hot cache directly" and its
data-flow figure: the compact selection feeds GPU attention.

Checks per step:
  * hc_attend (rows from the gathered bf16 buffer) and hc_attend_cached (rows
    from the slots, ring and host RAM, dequantised on the way) agree bit for
    bit;
  * both agree with the oracle's double-precision attention over the
    oracle's own gathered rows within |gpu - oracle| <= 4e-3 * max_i |v_i,d| +
    1e-6 per output value: the softmax weights are rounded to bf16 for the
    second matrix product (relative 2^-9 each, so at most 2^-9 of the largest
    value in a convex combination), and the scores are fp32 sums of exact
    bf16 products (about 1e-3 at most on this data);
  * steps that skip the bf16 buffer (d_out = NULL) still fill their slots.
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


def _val(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_attention(p, t, o_out, heads, layers=None, oracle_units=None, scale=SCALE):
    """Runs both attention paths after step t; o_out: the oracle's gathered
    rows of that step ([S, L, K, 576] or [S, L, Q, K, 576])."""
    import torch
    import oracle
    wl, Q = p.wl, p.Q
    q = W.queries(wl, t, heads, Q)
    d_q = torch.from_numpy(q.view(np.int16)).cuda()
    work, out = p.hc.attention_buffers(heads)
    cached = None
    if not p.fill_only:
        p.hc.attend(d_q, heads, scale, p.out, work, out)
        torch.cuda.synchronize()
        buf = out.cpu().numpy().copy()
    p.hc.attend_cached(d_q, heads, scale, work, out)
    torch.cuda.synchronize()
    cached = out.cpu().numpy()
    if not p.fill_only:
        assert np.array_equal(buf.view(np.uint32), cached.view(np.uint32)), \
            "buffer and slot paths differ at step %d" % t
    qq = q if Q > 1 else q[:, :, None]
    oo = o_out if Q > 1 else o_out[:, :, None]
    gg = cached if Q > 1 else cached[:, :, None]
    layers = range(wl.n_layers) if layers is None else layers
    worst = 0.0
    for s in range(wl.n_sessions):
        for l in layers:
            for qi in range(Q):
                ref = oracle.attend(qq[s, l, qi], oo[s, l, qi], scale)
                vmax = np.abs(_val(oo[s, l, qi][:, :512])).max(axis=0)
                err = np.abs(gg[s, l, qi].astype(np.float64) - ref)
                bound = 4e-3 * vmax[None, :] + 1e-6
                assert np.all(err <= bound), "step %d s %d l %d q %d: worst ratio %.3g" % (
                    t, s, l, qi, (err / bound).max())
                worst = max(worst, float((err / (vmax[None, :] + 1e-30)).max()))
    return worst


def _run(p, steps, heads, every=1, layers=None):
    from gpu_harness import say
    worst = 0.0
    for t in range(steps):
        g, o = p.step(t)
        p.compare(t, g, o)
        if t % every == 0 or t == steps - 1:
            worst = max(worst, check_attention(p, t, o[1], heads, layers))
    say("%s: attention within %.2e of max|v| (bound 4e-3)" % (p.wl.name, worst))


def test_attend_tiny():
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(steps=4))
    _run(p, 4, 64)
    p.close()


def test_attend_ragged_splits_two_head_groups_and_sessions():
    from gpu_harness import Pair
    wl = W.TINY.with_(name="attend_ragged", top_k=1000, cache_slots=2048, n_sessions=2,
                      n_layers=3, layers_per_select=2, steps=3, sigma_bias=(0.5, 0.5),
                      sigma_noise=(1.0, 1.0))
    p = Pair(wl)
    _run(p, 3, 128)
    p.close()


def test_scales_that_move_the_maximum_and_negative_scales():
    """The kernel keeps a reference maximum per head and raises it only when a
    64-row sub-chunk exceeds it by more than 2^8.  32 layers of top-2,048 give
    eight splits of 256 rows, four sub-chunks each.  At scale 1.0 this data's
    scores spread over hundreds of powers of two, so later sub-chunks often
    raise the maximum too; scale 1e-6 gives nearly equal weights, and a
    negative scale the softmax of negated scores.  Both paths bit for bit on
    every layer, three layers against the oracle."""
    from gpu_harness import Pair, say
    wl = W.TINY.with_(name="attend_scales", n_layers=32, layers_per_select=4, top_k=2048,
                      cache_slots=4096, steps=2)
    p = Pair(wl)
    for t in range(2):
        g, o = p.step(t)
        p.compare(t, g, o)
    for scale in (1.0, 1e-6, -SCALE):
        worst = check_attention(p, 1, o[1], 64, layers=[0, 13, 31], scale=scale)
        say("scale %g: attention within %.2e of max|v| (bound 4e-3)" % (scale, worst))
    p.close()


def test_largest_head_count():
    """4,096 heads (the largest hc_attend accepts): 64 head groups of one
    layer, both paths bit for bit, every head against the oracle."""
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(name="attend_4096_heads", steps=2))
    _run(p, 2, 4096)
    p.close()


def test_steps_without_the_bf16_buffer():
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(steps=6))
    p.fill_only = True
    _run(p, 6, 64)
    p.compare_state()
    p.close()


def test_mtp_round_duplicate_misses_read_host_ram():
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(steps=3), queries=4)
    _run(p, 3, 64)      # step 0: every row misses, three of four query rows read host RAM
    p.close()


def test_recent_ring_rows():
    from gpu_harness import RingPair
    p = RingPair(W.TINY.with_(steps=10), 16, 8, recent_boost=2.0)
    _run(p, 10, 64, every=3)
    p.close()


def test_model78_page_shape():
    """78 layers, history 50,023, 32,768 slots, top-2,048, 64 heads: both paths
    agree bit for bit on every layer; the oracle checks six layers."""
    from gpu_harness import Pair
    p = Pair(W.MODEL78_50K.with_(steps=3))
    _run(p, 3, 64, layers=[0, 1, 13, 38, 76, 77])
    p.close()


def test_invalid_attention_arguments_are_rejected():
    """Checked on the host before anything is enqueued (HC_E_INVAL, or
    HC_E_NOMEM for a scratch area that is too small): a call before the first
    step, heads not a multiple of 64, scratch or output not 16-byte aligned;
    a valid call afterwards still matches the buffer path."""
    import torch
    from cache_gather_amd import hc
    from gpu_harness import Pair
    p = Pair(W.TINY.with_(steps=1))
    heads = 64
    work, out = p.hc.attention_buffers(heads)
    q = torch.from_numpy(W.queries(p.wl, 0, heads, 1).view(np.int16)).cuda()
    st = torch.cuda.current_stream().cuda_stream

    def status(*args):
        try:
            hc.hc_attend_cached(p.hc.ctx, st, *args)
        except hc.HcError as e:
            return e.status
        return 0

    assert status(q, heads, SCALE, work, work.numel(), out) == -1      # no step yet
    g, o = p.step(0)
    p.compare(0, g, o)
    assert status(q, 96, SCALE, work, work.numel(), out) == -1         # heads % 64
    assert status(q, heads, SCALE, work, work.numel() - 1, out) == -2  # scratch too small
    assert status(q, heads, SCALE, work[4:], work.numel() - 4, out) == -1
    flat = torch.empty(out.numel() + 4, dtype=torch.float32, device="cuda")
    assert status(q, heads, SCALE, work, work.numel(), flat[1:]) == -1
    assert status(q, heads, SCALE, work, work.numel(), out) == 0
    torch.cuda.synchronize()
    cached = out.cpu().numpy().copy()
    p.hc.attend(q, heads, SCALE, p.out, work, out)
    torch.cuda.synchronize()
    assert np.array_equal(cached.view(np.uint32), out.cpu().numpy().view(np.uint32))
    p.close()
