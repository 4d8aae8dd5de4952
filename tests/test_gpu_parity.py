"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Everything must be bit-exact: selections, hit/miss/victim/eviction traces,
slot maps, hot-row bytes and the bf16 output buffer.
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
    maps = open("/proc/self/maps").read()
    assert "libhc.so" in maps, "the HIP library is not loaded"
    yield


def _pair(wl, **kw):
    from gpu_harness import Pair
    return Pair(wl, **kw)


def test_tiny_workload_every_step():
    p = _pair(W.TINY)
    p.run()
    p.close()


SMALL_CASES = [
    # name, S, L, R, H0, steps, C, K, sigma_b, sigma_n
    ("groups_ragged", 2, 5, 2, 700, 10, 96, 48, 0.5, 1.0),
    ("multi_chunk_tail", 1, 3, 3, 20011, 8, 700, 333, 0.3, 1.0),   # 3 scan chunks + ragged tail
    ("c_equals_k", 2, 2, 1, 3000, 12, 257, 257, 0.2, 1.0),
    ("k_one", 1, 2, 1, 500, 20, 4, 1, 0.2, 1.0),
    ("k_max", 1, 1, 1, 40000, 6, 5000, 4096, 1.0, 0.5),
    ("h_equals_k", 1, 1, 1, 2048, 1, 2048, 2048, 1.0, 1.0),
    ("many_sessions", 9, 1, 1, 9000, 6, 1100, 1000, 0.5, 1.0),
    ("wide_slots", 1, 1, 1, 90000, 6, 65536, 2048, 0.2, 1.0),
    # the LRU queue: compaction nearly every step with live and dead entries mixed
    ("lru_churn", 1, 2, 1, 6000, 60, 400, 300, 0.6, 1.0),
    # the LRU queue: long runs between compactions, evictions once the cache is full
    ("lru_long_queue", 1, 1, 1, 20000, 80, 2048, 64, 0.5, 1.0),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_configurations(case):
    name, S, L, R, H0, steps, C, K, sb, sn = case
    wl = W.Workload(name, S, L, R, H0, steps, C, K, (sb,) * S, (sn,) * S, 4242)
    p = _pair(wl)
    p.run()
    if name.startswith("lru_"):
        assert p.evictions > 0, "the case must evict to exercise the LRU queue"
    p.close()


@pytest.mark.parametrize("queries", [1, 2])
def test_step_that_takes_never_used_slots_and_evicts(queries):
    """C = 1.5 K with low overlap: the first step fills K slots, the next
    needs more than the C - K never-used slots left, so one step takes those
    (evicting nothing) and then evicts through the LRU queue.  The traces
    must show such a step, and every step stays bit-exact."""
    K = 1024 // queries
    wl = W.Workload("fill_then_evict_q%d" % queries, 1, 2, 1, 8000, 8, 3 * K * queries // 2, K,
                    (0.2,), (1.0,), 4243)
    p = _pair(wl, queries=queries)
    mixed = 0
    for t in range(wl.steps):
        g, o = p.step(t)
        p.compare(t, g, o)
        info = o[2][0]
        if info["n_evict"] > 0 and info["n_miss"] > info["n_evict"]:
            mixed += 1
    p.compare_state()
    assert mixed >= 1, "no step both filled never-used slots and evicted"
    p.close()


def test_unaligned_score_stride_uses_scalar_loads():
    wl = W.Workload("odd_stride", 2, 2, 2, 9001, 5, 600, 300, (0.5, 0.5), (1.0, 1.0), 99)
    p = _pair(wl, score_stride=wl.hcap + 3)
    p.run()
    p.close()


def _run_custom_scores(wl, make_scores):
    p = _pair(wl)
    for t in range(wl.steps):
        sc = np.zeros((wl.n_units, p.stride), np.float32)
        for u in range(wl.n_units):
            sc[u, :wl.hist0 + t] = make_scores(t, u, wl.hist0 + t)
        g, o = p.step(t, scores_np=sc)
        p.compare(t, g, o)
    p.compare_state()
    p.close()


def test_all_equal_scores_take_the_lowest_positions():
    wl = W.Workload("all_equal", 1, 2, 1, 5000, 4, 600, 512, (1.0,), (1.0,), 5)
    _run_custom_scores(wl, lambda t, u, h: np.full(h, 0.25, np.float32))


def test_heavy_ties_at_the_cut():
    wl = W.Workload("ties", 2, 1, 1, 30000, 6, 3000, 1500, (1.0, 1.0), (1.0, 1.0), 6)

    def mk(t, u, h):
        rng = np.random.default_rng((t, u))
        return (np.round(rng.standard_normal(h) * 4) / 4).astype(np.float32)
    _run_custom_scores(wl, mk)


def test_signed_zeros_infinities_and_nans():
    wl = W.Workload("ieee", 1, 1, 1, 3000, 4, 400, 300, (1.0,), (1.0,), 7)
    pnan = np.array([0x7FC00000, 0x7F800001, 0xFFC00000, 0xFFFFFFFF],
                    np.uint32).view(np.float32)

    def mk(t, u, h):
        rng = np.random.default_rng((t, 9))
        x = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf], np.float32), h)
        x[rng.integers(0, h, 40)] = rng.choice(pnan, 40)
        return x.astype(np.float32)
    _run_custom_scores(wl, mk)


def test_cut_jumping_between_steps_rescans_exactly():
    """Scores shifted far between steps move the cut bin outside the window
    predicted from the previous step; the select kernel then rebuilds its
    candidate lists from the scores.  Both paths must be exact."""
    wl = W.Workload("jumping_cut", 2, 2, 1, 20000, 8, 2600, 1300, (1.0, 1.0), (1.0, 1.0), 11)

    def mk(t, u, h):
        rng = np.random.default_rng((t, u, 5))
        x = rng.standard_normal(h).astype(np.float32)
        return (x * np.float32(1 + 3 * (t % 3)) + np.float32((-1) ** t * 40.0 * t)).astype(np.float32)
    _run_custom_scores(wl, mk)


@pytest.mark.parametrize("queries", [1, 2])
def test_many_units_with_flat_and_ordinary_scores(queries):
    """Sixteen sessions of 264,000 positions: 2,064 scan workgroups per query
    row, more than the chip holds in one resident round.  The even sessions'
    scores are flat, so every key lies inside the cut window and the select
    kernel ranks the whole history as entries; the odd sessions' are
    ordinary.  Every step stays bit-exact."""
    S = 16
    wl = W.Workload("many_units_q%d" % queries, S, 1, 1, 264000, 3, 512, 256, (1.0,) * S,
                    (1.0,) * S, 17)
    p = _pair(wl, queries=queries)
    for t in range(wl.steps):
        h = wl.hist0 + t
        sc = np.zeros((wl.n_units * queries, p.stride), np.float32)
        for uq in range(wl.n_units * queries):
            if (uq // queries) % 2 == 0:
                sc[uq, :h] = 0.5
            else:
                sc[uq, :h] = np.random.default_rng((t, uq, 3)).standard_normal(h)
        g, o = p.step(t, scores_np=sc)
        p.compare(t, g, o)
    p.compare_state()
    p.close()


def test_dequant_every_int8_with_every_finite_fp16_scale():
    """Rows covering all 256 int8 values against all 63,488 finite fp16 scales,
    gathered 2,048 rows per step through hc_step."""
    import oracle
    finite = np.arange(65536, dtype=np.int64)
    finite = finite[((finite >> 10) & 31) != 31]
    groups = np.repeat(finite, 4)                  # each scale for 4 x 64 int8 values
    quarter = np.tile(np.arange(4), finite.size)
    n_rows = -(-groups.size // 8)
    K = 2048
    steps = -(-n_rows // K)
    hcap = steps * K
    n_all = hcap + steps                            # the workload's Hcap is hist0 + steps
    latent = np.zeros((n_all, 8, 64), np.int8)
    scales = np.zeros((n_all, 8), np.uint16)
    q = (np.arange(64)[None, :] + 64 * quarter[:, None] - 128).astype(np.int8)   # [groups, 64]
    gi = np.arange(groups.size)
    latent[gi // 8, gi % 8, :] = q
    scales[gi // 8, gi % 8] = groups.astype(np.uint16)
    rows = np.zeros((n_all, 656), np.uint8)
    rows[:, :512] = latent.reshape(n_all, 512).view(np.uint8)
    rows[:, 512:528] = scales.astype("<u2").view(np.uint8).reshape(n_all, 16)
    rows[:, 528:] = np.random.default_rng(3).integers(0, 256, (n_all, 128), dtype=np.uint8)
    wl = W.Workload("dequant_all", 1, 1, 1, hcap, steps, K, K, (1.0,), (1.0,), 8)
    from gpu_harness import Pair
    p = Pair(wl, rows_fn=lambda s, l: rows)
    for t in range(steps):
        sc_t = np.zeros((1, p.stride), np.float32)
        sc_t[0, t * K:(t + 1) * K] = 1.0
        g, o = p.step(t, scores_np=sc_t, hist_len=np.array([hcap], np.uint64))
        p.compare(t, g, o)
        np.testing.assert_array_equal(g["sel"][0, 0], np.arange(t * K, (t + 1) * K))
        want = np.stack([oracle.dequant_row(rows[x]) for x in range(t * K, (t + 1) * K)])
        np.testing.assert_array_equal(g["out"][0, 0], want)
    p.close()


LIMIT_CASES = [
    # name, S, L, R, H0, steps, C, K, queries, sigma_b, sigma_n, sigma_draft, must_evict
    ("max_slots_max_topk", 1, 1, 1, 300000, 4, 262144, 4096, 1, 0.2, 1.0, None, False),
    # HC_MAX_QUERIES query rows of K = 512 fill HC_MAX_ROUND_ROWS = C; independent-looking
    # query rows (draft noise 3) make the round's union fill the cache by the fourth step
    ("max_queries_round_rows", 1, 2, 1, 9000, 6, 8192, 512, 16, 0.2, 1.0, 3.0, True),
    ("max_sessions", 256, 1, 1, 600, 4, 96, 64, 1, 0.5, 1.0, None, True),
    ("max_units", 16, 256, 1, 200, 4, 80, 48, 1, 0.3, 1.0, None, True),      # HC_MAX_UNITS = S * G
    ("many_layers", 1, 12000, 4, 40, 4, 16, 8, 1, 0.3, 1.0, None, True),     # 12,000 gather grid rows
]


@pytest.mark.parametrize("case", LIMIT_CASES, ids=[c[0] for c in LIMIT_CASES])
def test_configuration_limits(case):
    """The largest slot count with the largest top-K (HC_MAX_SLOTS,
    HC_MAX_TOPK), the largest number of query rows filling the largest round
    with C equal to it (HC_MAX_QUERIES, HC_MAX_ROUND_ROWS), the largest
    number of sessions (HC_MAX_SESSIONS) and of selection units (HC_MAX_UNITS),
    and 12,000 layers of one session (as many gather grid rows): every step
    bit-exact, then the end state."""
    name, S, L, R, H0, steps, C, K, Q, sb, sn, draft, must_evict = case
    wl = W.Workload(name, S, L, R, H0, steps, C, K, (sb,) * S, (sn,) * S, 4244)
    p = _pair(wl, queries=Q)
    for t in range(steps):
        sc = None if draft is None else p.scores.step(t, p.stride, queries=Q, sigma_draft=draft)
        g, o = p.step(t, scores_np=sc)
        p.compare(t, g, o)
    p.compare_state()
    if must_evict:
        assert p.evictions > 0, "the case must evict"
    p.close()


def test_history_beyond_4096_scan_segments():
    """8,400,000 positions: more than 4,096 chunks of 2,048, so the scan gives
    each workgroup two chunks (a segment of 4,096 positions, 2,051 segments)
    and the select kernel reads the longer segments.  One session and layer,
    small K and C; every step bit-exact, then the end state."""
    wl = W.Workload("long_8m", 1, 1, 1, 8400000, 3, 4096, 1024, (1.0,), (1.0,), 4245)
    p = _pair(wl)
    p.run()
    p.close()


def test_largest_recent_ring():
    """HC_MAX_RING_ROWS ring rows per layer with copyback batches of 8: every
    appended row stays in the ring, the copybacks still reach host RAM."""
    from gpu_harness import RingPair
    p = RingPair(W.TINY.with_(name="max_ring", steps=12), 65536, 8)   # HC_MAX_RING_ROWS
    p.run()
    p.close()
