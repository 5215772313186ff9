"""Pins for the oracle's importance scores (step 1).

The score is the observation-window attention of the AudioKV article
(section 1.2, the raw importance score that SnapKV-style methods rank by), with
softmax(q K^T / sqrt(d)) over the audio keys as written in the VoxZip digest's
decayed-eviction equation, pooled by the mean over window queries and the GQA
group.  The pins below are library routines and closed forms, not a retyping
of the oracle's loops.
"""
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import oracle as O


def test_single_query_matches_scipy_softmax():
    rng = np.random.default_rng(1)
    for L, d in [(1, 4), (7, 16), (64, 64), (200, 128)]:
        q = rng.standard_normal((1, d)) * 2.0
        k = rng.standard_normal((L, d))
        s = O.scores(q, k)
        ref = softmax(q[0] @ k.T / math.sqrt(d))
        np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-16)


def test_two_keys_logistic_closed_form():
    # q = e_0, k_0 = a e_0, k_1 = b e_0  =>  s_0 = logistic((a - b) / sqrt(d))
    for d in (1, 4, 64, 128):
        for a, b in [(3.0, 1.0), (-2.0, 5.0), (0.0, 0.0), (40.0, -40.0)]:
            q = np.zeros((1, d)); q[0, 0] = 1.0
            k = np.zeros((2, d)); k[0, 0] = a; k[1, 0] = b
            s = O.scores(q, k)
            p0 = expit((a - b) / math.sqrt(d))
            p1 = expit((b - a) / math.sqrt(d))
            np.testing.assert_allclose(s, [p0, p1], rtol=1e-13, atol=1e-300)


def test_mean_pooling_over_queries():
    # The pooled row is the average of the single-query rows.
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 32))
    k = rng.standard_normal((50, 32))
    pooled = O.scores(q, k)
    single = np.mean([softmax(q[i] @ k.T / math.sqrt(32)) for i in range(6)], axis=0)
    np.testing.assert_allclose(pooled, single, rtol=1e-13)


def test_distribution_invariants():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((17, 64)) * 3
    k = rng.standard_normal((333, 64))
    s = O.scores(q, k)
    assert np.all(s >= 0)
    assert abs(s.sum() - 1.0) < 1e-13


def test_identical_keys_give_uniform_row():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 16))
    k = np.tile(rng.standard_normal(16), (40, 1))
    np.testing.assert_allclose(O.scores(q, k), np.full(40, 1 / 40), rtol=1e-14)


def test_query_permutation_invariance_and_key_equivariance():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((9, 32))
    k = rng.standard_normal((77, 32))
    s = O.scores(q, k)
    np.testing.assert_allclose(O.scores(q[rng.permutation(9)], k), s, rtol=1e-13)
    perm = rng.permutation(77)
    np.testing.assert_allclose(O.scores(q, k[perm]), s[perm], rtol=1e-13)


def test_large_logits_do_not_overflow():
    # One key at logit +1000 relative to the rest: the row is one-hot there.
    d = 4
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((10, d)); k[3, 0] = 2000.0
    s = O.scores(q, k)
    assert np.all(np.isfinite(s))
    assert s[3] == pytest.approx(1.0, abs=1e-300)
    assert s.sum() == pytest.approx(1.0)


# ---------------------------------------------------------------------------
# Max pooling over query heads (the alternative reading of how a GQA group's
# attention rows are combined; C3 takes a max over a group's query heads)
# ---------------------------------------------------------------------------
def test_maxpool_two_heads_logistic_closed_form():
    # Head 0's queries are all x e_0, head 1's all y e_0; two keys e_0 and 0.
    # Each head's mean row is its single softmax row: (expit(x/sqrt d),
    # expit(-x/sqrt d)); the max over heads takes each key's larger one.
    from scipy.special import expit
    d, W = 16, 3
    for x, y in [(2.0, -1.0), (0.5, 7.0), (-3.0, -3.0)]:
        q = np.zeros((2 * W, d))
        q[:W, 0] = x
        q[W:, 0] = y
        k = np.zeros((2, d)); k[0, 0] = 1.0
        s = O.scores_maxpool(q, k, W)
        a = expit(np.array([x, y]) / math.sqrt(d))
        assert s[0] == pytest.approx(a.max(), rel=1e-13)
        assert s[1] == pytest.approx((1 - a).max(), rel=1e-13)


def test_maxpool_one_head_is_the_mean_and_dominates_the_mean():
    r = np.random.default_rng(8)
    q, k = r.standard_normal((32, 16)), r.standard_normal((50, 16))
    assert np.array_equal(O.scores_maxpool(q, k, 32), O.scores(q, k))
    q = r.standard_normal((4 * 8, 16))
    smax, smean = O.scores_maxpool(q, k, 8), O.scores(q, k)
    assert (smax >= smean - 1e-15).all()
    # heads in any order, queries within a head in any order
    perm = np.concatenate([np.arange(8) + 8 * h for h in (2, 0, 3, 1)])
    assert np.allclose(O.scores_maxpool(q[perm], k, 8), smax, atol=1e-15)
    perm = np.concatenate([r.permutation(8) + 8 * h for h in range(4)])
    assert np.allclose(O.scores_maxpool(q[perm], k, 8), smax, atol=1e-15)
