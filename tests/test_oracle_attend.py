"""Pins of the oracle's MLA decode attention (the consumer of the gather).

Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
section "Decision three: let the GPU manage the hot cache directly" and its
data-flow figure: the compact selection feeds GPU attention.  Reading
(absorbed MLA decode): per head, z_i = scale * <q, row_i> over the 576
values of each gathered row (512 latent + 64 RoPE), softmax over the K rows,
output = the softmax-weighted sum of the rows' 512 latent values.

Pins, none of which retypes the softmax:
  * one row: every head returns that row's latent values;
  * a zero query: every head returns the arithmetic mean of the rows;
  * two rows whose scores differ by exactly ln 3 (scale chosen so): weights
    3/4 and 1/4;
  * the RoPE values take part in the scores, the latent values alone in the
    output;
  * adding the same amount to every score (a shared RoPE component) changes
    nothing; permuting the rows changes nothing;
  * outputs lie within the rows' range; a score 1,000 above the rest selects
    its row (the largest score is subtracted before exponentiating).
"""
import math

import numpy as np
import pytest

import oracle


def bf16(x):
    """bf16 bit patterns of values that are exactly representable."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def val(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rows(rng, k):
    return bf16(rng.integers(-64, 64, (k, 576)).astype(np.float32) / 8)


def test_one_row_returns_it():
    rng = np.random.default_rng(1)
    rows = _rows(rng, 1)
    q = bf16(rng.integers(-8, 8, (4, 576)).astype(np.float32))
    out = oracle.attend(q, rows, 0.05)
    for h in range(4):
        np.testing.assert_array_equal(out[h], val(rows[0, :512]))


def test_zero_query_returns_the_mean():
    rng = np.random.default_rng(2)
    rows = _rows(rng, 37)
    q = np.zeros((3, 576), np.uint16)
    out = oracle.attend(q, rows, 0.7)
    want = val(rows[:, :512]).mean(axis=0)
    for h in range(3):
        np.testing.assert_allclose(out[h], want, rtol=0, atol=1e-12)


def test_scores_apart_by_ln3_weigh_three_to_one():
    rng = np.random.default_rng(3)
    rows = _rows(rng, 2)
    rows[:, 0] = bf16(np.array([2.0, 0.0]))
    rows[:, 1:] = np.where(np.arange(1, 576) < 512, rows[:, 1:], 0)  # no RoPE
    q = np.zeros((1, 576), np.uint16)
    q[0, 0] = bf16(np.array([1.0]))[0]
    out = oracle.attend(q, rows, math.log(3.0) / 2.0)   # z0 - z1 = ln 3
    want = 0.75 * val(rows[0, :512]) + 0.25 * val(rows[1, :512])
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)


def test_rope_counts_in_scores_not_in_output():
    rng = np.random.default_rng(4)
    rows = _rows(rng, 8)
    rows[:, 512:] = 0
    rows[3, 512] = bf16(np.array([64.0]))[0]         # only row 3 has RoPE
    q = np.zeros((1, 576), np.uint16)
    q[0, 512] = bf16(np.array([64.0]))[0]            # the query looks at RoPE only
    out = oracle.attend(q, rows, 1.0)                # row 3 scores 4,096 above the rest
    np.testing.assert_allclose(out[0], val(rows[3, :512]), rtol=0, atol=1e-12)


def test_shared_score_shift_and_row_order_change_nothing():
    rng = np.random.default_rng(5)
    rows = _rows(rng, 50)
    q = bf16(rng.integers(-4, 4, (2, 576)).astype(np.float32) / 4)
    base = oracle.attend(q, rows, 0.03)
    shifted_rows = rows.copy()
    shifted_rows[:, 575] = bf16(np.full(50, 3.0))     # same RoPE value in every row
    shifted_q = q.copy()
    shifted_q[:, 575] = bf16(np.full(2, 5.0))         # adds 15 * scale to every score
    base2 = oracle.attend(q, np.where(np.arange(576) == 575, 0, rows).astype(np.uint16), 0.03)
    shifted = oracle.attend(shifted_q, shifted_rows, 0.03)
    np.testing.assert_allclose(shifted, base2, rtol=1e-12, atol=1e-12)
    perm = rng.permutation(50)
    np.testing.assert_allclose(oracle.attend(q, rows[perm], 0.03), base, rtol=1e-12, atol=1e-12)


def test_outputs_are_convex_combinations_and_large_scores_stay_finite():
    rng = np.random.default_rng(6)
    rows = _rows(rng, 200)
    q = bf16(rng.integers(-8, 8, (5, 576)).astype(np.float32))
    out = oracle.attend(q, rows, 0.2)
    v = val(rows[:, :512])
    assert np.all(out >= v.min(axis=0) - 1e-9) and np.all(out <= v.max(axis=0) + 1e-9)
    # one row scores 1,000 above all others: exp would overflow without the shift
    rows2 = rows.copy()
    rows2[:, 1:] = np.where(np.arange(1, 576) < 512, rows2[:, 1:], 0)
    rows2[:, 0] = 0
    rows2[17, 0] = bf16(np.array([1000.0]))[0]
    q2 = np.zeros((1, 576), np.uint16)
    q2[0, 0] = bf16(np.array([1.0]))[0]
    out2 = oracle.attend(q2, rows2, 1.0)
    assert np.all(np.isfinite(out2))
    np.testing.assert_allclose(out2[0], val(rows2[17, :512]), rtol=0, atol=1e-12)
