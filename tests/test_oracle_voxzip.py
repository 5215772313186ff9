"""Pins of the decayed-eviction oracle (oracle/voxzip.py) against closed
forms, invariants and brute force -- not against a retyped formula.

VoxZip digest page, method overview, "Temporally Decayed KV Cache Eviction"
(update equation and concatenation rule; gamma, T and the 20 % recent window
from the details list)."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import voxzip as VZ


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# softmax rows
# ---------------------------------------------------------------------------
def test_identical_keys_give_uniform_rows():
    r = rng(1)
    k = np.tile(r.standard_normal(16), (37, 1))
    p = VZ.attention_rows(r.standard_normal((3, 16)), k)
    assert np.allclose(p, 1.0 / 37, rtol=0, atol=1e-15)


def test_two_keys_logistic_with_sqrt_d_scale():
    # q = x e_0, k_0 = e_0, k_1 = 0: logits x / sqrt(d) and 0, so
    # p_0 = logistic(x / sqrt(d)); a wrong scale or axis fails this.
    d = 64
    for x in (-7.0, -0.3, 0.0, 2.5, 11.0):
        q = np.zeros((1, d)); q[0, 0] = x
        k = np.zeros((2, d)); k[0, 0] = 1.0
        p = VZ.attention_rows(q, k)
        assert p[0, 0] == pytest.approx(expit(x / math.sqrt(d)), rel=1e-14)
        assert p[0, 1] == pytest.approx(expit(-x / math.sqrt(d)), rel=1e-14)


def test_rows_normalise_over_keys_not_queries():
    # Adding one vector to every key shifts each query's logits by a
    # constant: the softmax over keys cannot change.  A softmax taken over
    # the query axis would.
    r = rng(2)
    q, k = r.standard_normal((5, 32)), r.standard_normal((50, 32))
    shift = 3.0 * r.standard_normal(32)
    assert np.allclose(VZ.attention_rows(q, k), VZ.attention_rows(q, k + shift), atol=1e-13)
    p = VZ.attention_rows(q, k)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert (p >= 0).all()


def test_query_head_order_does_not_matter():
    r = rng(3)
    q, k = r.standard_normal((7, 32)), r.standard_normal((40, 32))
    a = VZ.accumulate(np.zeros(39), q, k, 0.95)
    b = VZ.accumulate(np.zeros(39), q[::-1], k, 0.95)
    assert np.allclose(a, b, atol=1e-15)


# ---------------------------------------------------------------------------
# decayed accumulation
# ---------------------------------------------------------------------------
def test_single_row_cache():
    r = rng(4)
    A = VZ.accumulate(np.zeros(0), r.standard_normal((2, 8)), r.standard_normal((1, 8)), 0.95)
    assert A.tolist() == [1.0]


def test_mass_balance():
    # Each step adds one unit of attention mass: sum A(t) = gamma sum A(t-1) + 1.
    r = rng(5)
    for gamma in (0.0, 0.5, 0.95, 1.0):
        a_prev = r.exponential(size=63)
        A = VZ.accumulate(a_prev, r.standard_normal((4, 16)), r.standard_normal((64, 16)), gamma)
        assert A.sum() == pytest.approx(gamma * a_prev.sum() + 1.0, rel=1e-13)


def test_decay_closed_form_over_steps():
    # Identical keys: every step's row is 1/n_s on each of its n_s rows, so
    # after steps s = 1..t (cache growing by one row per step, no eviction)
    # A[j] = sum over steps that saw row j of gamma^(t - s) / n_s.
    r = rng(6)
    d, gamma, n0, steps = 16, 0.9, 5, 6
    row = r.standard_normal(d)
    A = np.zeros(n0 - 1)
    for s in range(steps):
        n = n0 + s
        A = VZ.accumulate(A, r.standard_normal((3, d)), np.tile(row, (n, 1)), gamma)
    t = steps - 1
    want = np.zeros(n0 + t)
    for s in range(steps):
        n = n0 + s
        want[:n] += gamma ** (t - s) / n
    assert np.allclose(A, want, rtol=1e-13, atol=0)


def test_new_row_gets_no_decayed_term():
    r = rng(7)
    q, k = r.standard_normal((2, 8)), r.standard_normal((10, 8))
    a1 = VZ.accumulate(np.full(9, 5.0), q, k, 0.95)
    a0 = VZ.accumulate(np.zeros(9), q, k, 0.95)
    assert a1[-1] == a0[-1]
    assert np.allclose(a1[:-1] - a0[:-1], 0.95 * 5.0, atol=1e-13)


# ---------------------------------------------------------------------------
# eviction
# ---------------------------------------------------------------------------
def test_split_of_the_page_defaults():
    # T = 4 sinks, recent window 20 % of the budget.
    assert VZ.split(8192, 4, 0.2) == (4, 1638, 6550)
    assert VZ.split(200, 4, 0.2) == (4, 40, 156)
    assert VZ.split(10, 4, 0.2) == (4, 2, 4)
    assert VZ.split(6, 4, 0.2) == (4, 1, 1)
    assert VZ.split(4, 4, 0.2) == (4, 0, 0)
    with pytest.raises(ValueError):
        VZ.split(5, 4, 0.5)


def test_no_eviction_within_budget():
    A = rng(8).random(50)
    assert VZ.evict(A, 50, 4, 0.2).tolist() == list(range(50))
    assert VZ.evict(A, 80, 4, 0.2).tolist() == list(range(50))


def test_eviction_matches_exhaustive_search():
    # Distinct values: the kept middle set is the N-subset of largest sum.
    r = rng(9)
    for n, B, T, frac in [(12, 8, 2, 0.25), (11, 9, 1, 0.3), (10, 6, 0, 0.0), (9, 7, 3, 0.2)]:
        A = r.permutation(n).astype(float) + r.random(n) * 0.1
        M = math.floor(frac * B)
        N = B - T - M
        mid = list(range(T, n - M))
        best = max(itertools.combinations(mid, N), key=lambda c: sum(A[list(c)]))
        want = list(range(T)) + sorted(best) + list(range(n - M, n))
        assert VZ.evict(A, B, T, frac).tolist() == want


def test_eviction_structure_and_ties():
    # Equal values: the lowest middle positions win; sinks and the recent
    # window always stay; -0.0 equals +0.0.
    A = np.zeros(30)
    A[4] = -0.0                                   # not below +0.0
    kept = VZ.evict(A, 12, 4, 0.25)               # M = 3, N = 5
    assert kept.tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 8, 27, 28, 29]
    A = np.ones(30)
    A[20] = 2.0
    kept = VZ.evict(A, 12, 4, 0.25)
    assert kept.tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 20, 27, 28, 29]
    # sinks and recent rows are kept even when their A is the smallest
    A = np.arange(30, dtype=float)[::-1].copy()
    kept = VZ.evict(A, 12, 4, 0.25)
    assert kept[:4].tolist() == [0, 1, 2, 3] and kept[-3:].tolist() == [27, 28, 29]
    assert kept[4:9].tolist() == [4, 5, 6, 7, 8]


def test_step_gathers_k_v_and_a_with_the_same_positions():
    r = rng(10)
    n, d = 40, 8
    q, k, v = r.standard_normal((2, d)), r.standard_normal((n, d)), r.standard_normal((n, d))
    out = VZ.step(q, k, v, r.random(n - 1), 25)
    kept = out["kept"]
    assert len(kept) == 25 and np.all(np.diff(kept) > 0)
    assert np.array_equal(out["k_out"], k[kept]) and np.array_equal(out["v_out"], v[kept])
    assert np.array_equal(out["a_out"], out["A"][kept])
