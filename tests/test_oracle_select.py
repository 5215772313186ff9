"""Pins for the oracle's per-head selection (step 4).

The kept set is the b - w candidates with the largest smoothed score (AudioKV
article, section 2.2: SSS feeds the token selection) plus the w most recent
positions (section 3.1: the local window of w = 32 tokens).  Keeping the
top-weighted positions maximises the retained attention mass (C3 digest,
the output-error identity).  Pins: exhaustive subset search and order
invariants.
"""
import itertools

import numpy as np
import pytest

from oracle import oracle as O


def brute_force(vals, w, b):
    L = len(vals)
    cand = range(L - w)
    k = b - w
    best = None
    for sub in itertools.combinations(cand, k):
        tot = sum(vals[j] for j in sub)
        key = (-tot, sub)          # max sum, then lexicographically smallest
        if best is None or key < best:
            best = key
    chosen = list(best[1]) if best else []
    return chosen + list(range(L - w, L))


@pytest.mark.parametrize("seed", range(30))
def test_exhaustive_subset_search_small_rows(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 13))
    w = int(rng.integers(0, min(L, 3) + 1))
    b = int(rng.integers(w, L + 1))
    vals = rng.integers(-3, 4, L).astype(float)   # small integers: many ties, exact sums
    got = O.select(vals, w, b).tolist()
    assert got == brute_force(vals.tolist(), w, b)


def test_order_invariants_on_large_random_row():
    rng = np.random.default_rng(99)
    L, w, b = 4096, 32, 1500
    vals = np.round(rng.random(L), 3)              # ties at 3 decimals
    kept = O.select(vals, w, b)
    assert len(kept) == b
    assert np.all(np.diff(kept) > 0)
    assert kept[-w:].tolist() == list(range(L - w, L))
    sel = kept[:-w]
    dropped = np.setdiff1d(np.arange(L - w), sel)
    assert vals[sel].min() >= vals[dropped].max()
    thr = vals[sel].min()
    # among positions equal to the threshold, the kept ones are the lowest
    tied = np.flatnonzero(vals[:L - w] == thr)
    kept_tied = np.intersect1d(tied, sel)
    assert kept_tied.tolist() == tied[:len(kept_tied)].tolist()


def test_signed_zeros_are_equal():
    vals = np.array([0.0, -0.0, 0.0, -0.0, 1.0, 0.5])
    assert O.select(vals, 1, 3).tolist() == [0, 4, 5]
    vals = np.array([-0.0, 0.0, 1.0])
    assert O.select(vals, 0, 2).tolist() == [0, 2]


def test_degenerate_budgets():
    vals = np.random.default_rng(1).random(50)
    assert O.select(vals, 32, 32).tolist() == list(range(18, 50))
    assert O.select(vals, 32, 50).tolist() == list(range(50))
    assert O.select(vals, 0, 0).tolist() == []
