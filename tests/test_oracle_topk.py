"""Pins of the oracle's exact top-K selection.

The DSA indexer keeps the top 2,048 history positions by score (page "From 1M
Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading", section "Separate
historical capacity from the current working set"); the exact selection has
to stay on the GPU path, since a selection differing near the cutoff changed
the generated text (section "Decision one: should the CPU store history and
run the indexer?").  Reading taken: rank by IEEE-754 totalOrder (so -0 < +0),
ties to the lower position, emit positions in ascending order.

References that share nothing with the oracle's code:
  * a pairwise rank count: p is selected iff fewer than K positions rank above
    it (score greater, or equal with a lower position);
  * numpy.lexsort on (position, -score) for larger inputs without +-0 / NaN;
  * values the IEEE ordering fixes by hand (signed zeros, infinities, NaNs).
"""
import numpy as np
import pytest

import oracle


def rank_count_topk(scores, k):
    """Brute force: count, for every p, the positions ranking above it."""
    s = np.asarray(scores, np.float64)
    h = s.size
    greater = s[None, :] > s[:, None]                       # [p, q]: q beats p
    tie_lower = (s[None, :] == s[:, None]) & (np.arange(h)[None, :] < np.arange(h)[:, None])
    above = (greater | tie_lower).sum(axis=1)
    return np.flatnonzero(above < k).astype(np.int32)


def check_invariants(scores, k, sel):
    s = np.asarray(scores, np.float32)
    assert sel.size == k
    assert np.all(np.diff(sel) > 0)                          # ascending, distinct
    chosen = np.zeros(s.size, bool)
    chosen[sel] = True
    worst = s[sel].min()
    assert np.all(s[~chosen] <= worst)
    # equal to the cutoff score only at a higher position than every chosen tie
    ties_out = np.flatnonzero(~chosen & (s == worst))
    ties_in = sel[s[sel] == worst]
    if ties_out.size:
        assert ties_out.min() > ties_in.max()


@pytest.mark.parametrize("seed", range(12))
def test_random_against_rank_count(seed):
    rng = np.random.default_rng(seed)
    h = int(rng.integers(1, 600))
    k = int(rng.integers(1, h + 1))
    scores = rng.standard_normal(h).astype(np.float32)
    sel = oracle.topk(scores, k)
    np.testing.assert_array_equal(sel, rank_count_topk(scores, k))
    check_invariants(scores, k, sel)


@pytest.mark.parametrize("quantum", [1.0, 0.125])
@pytest.mark.parametrize("seed", range(6))
def test_heavy_ties_against_rank_count(seed, quantum):
    rng = np.random.default_rng(100 + seed)
    h = int(rng.integers(50, 700))
    k = int(rng.integers(1, h + 1))
    # + 0.0 turns the -0.0 that rounding makes into +0.0: the pairwise float
    # reference treats -0 == +0, totalOrder does not (pinned separately below)
    scores = (np.round(rng.standard_normal(h) / quantum) * quantum + 0.0).astype(np.float32)
    sel = oracle.topk(scores, k)
    np.testing.assert_array_equal(sel, rank_count_topk(scores, k))
    check_invariants(scores, k, sel)


def test_all_equal_takes_the_lowest_positions():
    for h, k in [(1, 1), (10, 3), (1000, 256), (4097, 4096)]:
        sel = oracle.topk(np.full(h, 0.5, np.float32), k)
        np.testing.assert_array_equal(sel, np.arange(k))


def test_k_equals_h_and_h_equals_k_plus_one():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(300).astype(np.float32)
    np.testing.assert_array_equal(oracle.topk(s, 300), np.arange(300))
    s2 = s[:257]
    drop = int(np.argmin(s2))
    np.testing.assert_array_equal(oracle.topk(s2, 256), np.delete(np.arange(257), drop))


def test_k_one_is_the_first_maximum():
    s = np.array([1.0, 3.0, -2.0, 3.0, 0.0], np.float32)
    np.testing.assert_array_equal(oracle.topk(s, 1), [1])


def test_ieee_total_order_by_hand():
    # totalOrder, descending: +NaN > +Inf > 1 > +0 > -0 > -Inf > -NaN
    pnan = np.array([0x7FC00000], np.uint32).view(np.float32)[0]
    nnan = np.array([0xFFC00000], np.uint32).view(np.float32)[0]
    s = np.array([-0.0, 1.0, nnan, np.inf, 0.0, -np.inf, pnan], np.float32)
    order = [6, 3, 1, 4, 0, 5, 2]             # positions by descending rank
    for k in range(1, 8):
        np.testing.assert_array_equal(oracle.topk(s, k), np.sort(order[:k]))


def test_signed_zero_breaks_what_would_otherwise_be_a_tie():
    s = np.array([-0.0, -0.0, 0.0, -1.0], np.float32)
    np.testing.assert_array_equal(oracle.topk(s, 1), [2])     # +0 above both -0
    np.testing.assert_array_equal(oracle.topk(s, 2), [0, 2])  # then the lower -0


@pytest.mark.parametrize("h,k", [(50023, 2048), (200_000, 2048), (4096, 256)])
def test_large_against_lexsort(h, k):
    rng = np.random.default_rng(h)
    bias = rng.standard_normal(h).astype(np.float32)
    scores = (bias + np.float32(0.3) * rng.standard_normal(h).astype(np.float32))
    scores[rng.integers(0, h, 50)] = scores[rng.integers(0, h, 50)]   # plant exact ties
    pos = np.arange(h)
    want = np.sort(np.lexsort((pos, -scores.astype(np.float64)))[:k])
    sel = oracle.topk(scores, k)
    np.testing.assert_array_equal(sel, want)
    check_invariants(scores, k, sel)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.topk(np.zeros(4, np.float32), 5)
    with pytest.raises(ValueError):
        oracle.topk(np.zeros(4, np.float32), 0)
