"""Pins of the learned-indexer oracle (``oracle/qsa_indexer.py``) against facts fixed by the mathematics.

- a worked example small enough to do by hand, for every aggregation;
- linearity: projecting then averaging a block's keys equals averaging (the
  pinned compression oracle) then projecting;
- identity projections with the sum aggregation reproduce the pinned default
  block scores;
- max over identical heads is any one head's score; a single head makes max,
  sum and softmax rank the candidates alike;
- softmax aggregation: the group's scores sum to the number of heads, and a
  constant added to one head's scores changes nothing;
- plain-Python loops (no matrix products) agree on random tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import qsa_indexer as I
from oracle import qsa_oracle as O


def test_worked_example_by_hand():
    # two heads, three candidates, identity projections in two dimensions, unit scale
    eye = np.eye(2)
    k_idx = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    q = np.array([[2.0, 0.0], [0.0, 1.0]])
    per_head = I.head_scores(q, eye, k_idx, 3, 1.0)
    assert per_head.tolist() == [[2.0, 0.0], [0.0, 1.0], [2.0, 1.0]]
    assert I.indexer_scores(q, eye, k_idx, 3, 1.0, I.AGG_SUM).tolist() == [2.0, 1.0, 3.0]
    assert I.indexer_scores(q, eye, k_idx, 3, 1.0, I.AGG_MAX).tolist() == [2.0, 1.0, 2.0]
    e, e2 = math.e, math.e ** 2
    want = [e2 / (2 * e2 + 1) + 1 / (1 + 2 * e),   # head 0 sees (2, 0, 2), head 1 sees (0, 1, 1)
            1 / (2 * e2 + 1) + e / (1 + 2 * e),
            e2 / (2 * e2 + 1) + e / (1 + 2 * e)]
    got = I.indexer_scores(q, eye, k_idx, 3, 1.0, I.AGG_SOFTMAX)
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # the selections these scores make (own block 3 forced, two slots)
    assert O.select_in_frame(I.indexer_scores(q, eye, k_idx, 3, 1.0, I.AGG_SUM), 3, 3, 3) == [0, 2, 3]
    assert O.select_in_frame(I.indexer_scores(q, eye, k_idx, 3, 1.0, I.AGG_MAX), 3, 3, 3) == [0, 2, 3]  # tie: smaller id
    assert O.select_in_frame(got, 3, 3, 3) == [0, 2, 3]


def test_default_indexer_scale_by_hand():
    """The indexer's default scale is 1/sqrt(dim): 1/8 for 64 dimensions, 1/4 for 16, and for 128 the
    value whose square times 128 is 1. A worked example with the default scale: two identity-projected
    heads in a 16-dimensional indexer space scoring one candidate."""
    assert I.default_indexer_scale(64) == 0.125
    assert I.default_indexer_scale(16) == 0.25
    s128 = I.default_indexer_scale(128)
    assert abs(s128 * s128 * 128 - 1.0) < 4e-16 and 0.0883 < s128 < 0.0884
    eye = np.eye(16)
    q = np.zeros((2, 16))
    q[0, 0], q[1, 3] = 2.0, -1.0
    k_idx = np.zeros((1, 16))
    k_idx[0, 0], k_idx[0, 3] = 3.0, 4.0
    per_head = I.head_scores(q, eye, k_idx, 1, I.default_indexer_scale(16))
    # head 0: 2 * 3 / 4 = 1.5; head 1: -1 * 4 / 4 = -1
    assert per_head.tolist() == [[1.5, -1.0]]
    assert I.indexer_scores(q, eye, k_idx, 1, I.default_indexer_scale(16), I.AGG_SUM).tolist() == [0.5]
    assert I.indexer_scores(q, eye, k_idx, 1, I.default_indexer_scale(16), I.AGG_MAX).tolist() == [1.5]


def test_project_then_average_equals_average_then_project():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((2, 3, 100, 16))
    W = rng.standard_normal((16, 8))
    got = I.indexer_keys(K, W, 8)
    want = O.compress_keys(K, 8) @ W
    assert got.shape == (2, 3, 12, 8)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_identity_projection_sum_matches_default_scores():
    rng = np.random.default_rng(2)
    d, G, nb = 32, 4, 40
    q = rng.standard_normal((G, d))
    kc = rng.standard_normal((nb, d))
    got = I.indexer_scores(q, np.eye(d), kc, nb, 0.25, I.AGG_SUM)
    want = O.block_scores(q, kc, nb, 0.25)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_max_of_identical_heads_and_single_head_rankings():
    rng = np.random.default_rng(3)
    d, d_idx, nb = 16, 8, 30
    W = rng.standard_normal((d, d_idx))
    kc = rng.standard_normal((nb, d_idx))
    one = rng.standard_normal((1, d))
    same = np.repeat(one, 4, axis=0)
    s1 = I.indexer_scores(one, W, kc, nb, 0.5, I.AGG_SUM)
    assert np.allclose(I.indexer_scores(same, W, kc, nb, 0.5, I.AGG_MAX), s1, rtol=0, atol=1e-12)
    assert np.allclose(I.indexer_scores(same, W, kc, nb, 0.5, I.AGG_SUM), 4 * s1, rtol=1e-12, atol=1e-12)
    picks = {agg: O.select_in_frame(I.indexer_scores(one, W, kc, nb, 0.5, agg), nb, nb, 9)
             for agg in (I.AGG_SUM, I.AGG_MAX, I.AGG_SOFTMAX)}
    assert picks[I.AGG_SUM] == picks[I.AGG_MAX] == picks[I.AGG_SOFTMAX]


def test_softmax_aggregation_invariants():
    rng = np.random.default_rng(4)
    per_head = rng.standard_normal((50, 8)) * 3
    agg = I.aggregate(per_head, I.AGG_SOFTMAX)
    assert abs(agg.sum() - 8.0) < 1e-12
    assert (agg > 0).all()
    shifted = per_head.copy()
    shifted[:, 3] += 123.0
    assert np.allclose(I.aggregate(shifted, I.AGG_SOFTMAX), agg, rtol=1e-12, atol=1e-15)
    assert I.aggregate(per_head[:0], I.AGG_SOFTMAX).shape == (0,)
    with pytest.raises(ValueError):
        I.aggregate(per_head, 7)


@pytest.mark.parametrize("agg", [I.AGG_SUM, I.AGG_MAX, I.AGG_SOFTMAX])
def test_plain_loops_agree(agg):
    rng = np.random.default_rng(5 + agg)
    d, d_idx, G, Bs, N = 6, 4, 3, 2, 14
    K = rng.standard_normal((N, d))
    W_k = rng.standard_normal((d, d_idx))
    W_q = rng.standard_normal((d, d_idx))
    q = rng.standard_normal((G, d))
    nb = N // Bs
    # projected keys averaged per block, loop by loop
    kidx = [[sum(sum(K[c * Bs + u][i] * W_k[i][e] for i in range(d)) for u in range(Bs)) / Bs for e in range(d_idx)]
            for c in range(nb)]
    assert np.allclose(I.indexer_keys(K, W_k, Bs), kidx, rtol=1e-12, atol=1e-12)
    qi = [[sum(q[j][i] * W_q[i][e] for i in range(d)) for e in range(d_idx)] for j in range(G)]
    scale = 0.5
    s = [[scale * sum(qi[j][e] * kidx[c][e] for e in range(d_idx)) for j in range(G)] for c in range(nb)]
    if agg == I.AGG_SUM:
        want = [sum(row) for row in s]
    elif agg == I.AGG_MAX:
        want = [max(row) for row in s]
    else:
        want = [0.0] * nb
        for j in range(G):
            m = max(s[c][j] for c in range(nb))
            z = sum(math.exp(s[c][j] - m) for c in range(nb))
            for c in range(nb):
                want[c] += math.exp(s[c][j] - m) / z
    got = I.indexer_scores(q, W_q, np.array(kidx), nb, scale, agg)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
