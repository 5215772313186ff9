"""Pins for the oracle's head-aware budget (step 3).

AudioKV article, section 3.1: b_{l,h} = w + r + B_score * S_{l,h} / sum S,
w = 32 local window, r the base share, B_score the rest; defaults from the
section 5.1 config block.  Pins: hand-worked cases (tests/golden), the exact
rational computation of the same apportionment, and the invariants that the
budgets sum exactly to N * kbar and respect their bounds.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "budget_hand.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    b = O.budget(case["S"], case["L"], case["retention"], case["base_ratio"], case["window"])
    assert b.tolist() == case["budgets"]


@pytest.mark.parametrize("case", _golden()["infeasible"], ids=lambda c: c["name"])
def test_infeasible_cases_rejected(case):
    rc = O.budget_rc(case["S"], case["L"], case["retention"], case["base_ratio"], case["window"])
    assert rc == -2


def exact_budget(S, L, retention, base_ratio, w):
    """Largest-remainder water-filling in exact rational arithmetic."""
    S = [Fraction(float(x)) for x in np.asarray(S, dtype=np.float32)]
    n = len(S)
    # kbar and r are defined by fp64 products (the parameters are fp64);
    # everything after them is exact here.
    kbar = math.floor(float(retention) * L)
    if kbar >= L:
        return [L] * n, None
    r = math.floor(float(base_ratio) * kbar)
    fixed = w + r
    R = n * kbar - n * fixed
    cap = L - fixed
    active = set(range(n))
    extra = [0] * n
    while True:
        tot = sum(S[u] for u in active)
        q = {u: (R * S[u] / tot if tot > 0 else Fraction(R, len(active))) for u in active}
        C = [u for u in active if q[u] >= cap]
        if not C:
            break
        for u in C:
            extra[u] = cap
            active.discard(u)
        R -= cap * len(C)
    fl = {u: math.floor(q[u]) for u in active}
    deficit = R - sum(fl.values())
    order = sorted(active, key=lambda u: (-(q[u] - fl[u]), u))
    for u in active:
        extra[u] = fl[u]
    for u in order[:deficit]:
        extra[u] += 1
    # smallest gap between distinct fractional parts, to know whether fp64
    # can be expected to rank them identically
    fr = sorted({q[u] - fl[u] for u in active})
    gap = min((b - a for a, b in zip(fr, fr[1:])), default=Fraction(1))
    return [fixed + e for e in extra], gap


def _random_cases(seed, count):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        n = int(rng.integers(1, 40))
        L = int(rng.choice([64, 100, 1024, 4096, 8192, 32768, 65536]))
        ret = float(rng.uniform(0.05, 1.0))
        base = float(rng.choice([0.0, 0.25, 0.5, 0.7]))
        kind = rng.integers(0, 4)
        if kind == 0:
            S = rng.uniform(0, 1, n)
        elif kind == 1:
            S = np.where(rng.random(n) < 0.2, rng.uniform(0.6, 1, n), rng.uniform(0, 0.2, n))
        elif kind == 2:
            S = np.zeros(n)
        else:
            S = rng.integers(0, 4, n).astype(float)
        yield S.astype(np.float32), L, ret, base


def test_matches_exact_rational_apportionment():
    checked = 0
    for S, L, ret, base in _random_cases(20, 400):
        if O.budget_rc(S, L, ret, base, 32) != 0:
            continue
        want, gap = exact_budget(S, L, ret, base, 32)
        if gap is not None and gap < Fraction(1, 10**9):
            continue  # near-tied remainders: fp64 may legitimately rank them apart
        assert O.budget(S, L, ret, base, 32).tolist() == want
        checked += 1
    assert checked > 200


def test_sum_and_bounds_invariants():
    for S, L, ret, base in _random_cases(21, 400):
        rc = O.budget_rc(S, L, ret, base, 32)
        kbar = math.floor(ret * L)
        r = math.floor(base * kbar)
        if kbar < L and (L <= 32 or 32 + r > kbar):
            assert rc == -2
            continue
        assert rc == 0
        b = O.budget(S, L, ret, base, 32)
        n = len(S)
        if kbar >= L:
            assert np.all(b == L)
            continue
        assert int(b.sum()) == n * kbar
        assert np.all(b >= 32 + r) and np.all(b <= L)


def test_monotone_in_head_score():
    for S, L, ret, base in _random_cases(22, 200):
        if O.budget_rc(S, L, ret, base, 32) != 0:
            continue
        b = O.budget(S, L, ret, base, 32)
        order = np.argsort(S, kind="stable")
        # a higher score never gets a smaller budget (one unit of slack for
        # equal scores, whose remainders tie and go to the lower index)
        for a, c in zip(order, order[1:]):
            if S[c] > S[a]:
                assert b[c] >= b[a]
            else:
                assert abs(int(b[c]) - int(b[a])) <= 1


def test_uniform_scores_differ_by_at_most_one_lower_index_first():
    for n in (1, 3, 7, 112, 192):
        b = O.budget(np.full(n, 0.3, np.float32), 8192, 0.6, 0.5, 32)
        assert b.max() - b.min() <= 1
        assert np.all(np.diff(b) <= 0)
        assert int(b.sum()) == n * math.floor(0.6 * 8192)


def test_single_head_gets_exactly_kbar():
    for L, ret in [(1024, 0.6), (32768, 0.4), (65536, 0.2)]:
        assert O.budget([0.7], L, ret).tolist() == [math.floor(ret * L)]


# ---------------------------------------------------------------------------
# One budget pool per layer (the alternative reading of AudioKV section 3.1:
# the score-proportional share split among a layer's heads only)
# ---------------------------------------------------------------------------
class _Prob:
    def __init__(self, S, lengths, retention, base_ratio=0.5, window=4, pool=1):
        NL, H = np.asarray(S).shape
        self.cfg = type("C", (), dict(n_layers=NL, n_kv_heads=H, n_seq=len(lengths),
                                      base_ratio=base_ratio, window=window, budget_pool=pool))()
        self.hdr = type("H", (), dict(head_scores=np.asarray(S, np.float32),
                                      lengths=np.asarray(lengths), retention=np.asarray(retention)))()


def test_layer_pool_hand_case():
    # L = 100, retention 0.5 -> kbar 50; w = 4, base_ratio 0.5 -> r = 25,
    # fixed = 29, cap = 71.  Layer 0, S = (1, 3): R = 2*50 - 2*29 = 42,
    # quotas 10.5 and 31.5, floors 10 + 31 = 41, one left over, equal
    # remainders -> the lower head: (11, 31) -> budgets (40, 60).  Layer 1,
    # S = (0, 0): uniform 21 each -> (50, 50).  One pool over all four heads
    # instead: R = 84 split 21 / 63 / 0 / 0 -> (50, 92, 29, 29).
    S = [[1.0, 3.0], [0.0, 0.0]]
    b_layer, off = O.problem_budgets(_Prob(S, [100], [0.5], pool=1))
    assert b_layer.tolist() == [40, 60, 50, 50]
    assert off.tolist() == [0, 40, 100, 150, 200]
    b_seq, _ = O.problem_budgets(_Prob(S, [100], [0.5], pool=0))
    assert b_seq.tolist() == [50, 92, 29, 29]


def test_layer_pool_sums_per_layer_and_single_layer_equals_sequence_pool():
    r = np.random.default_rng(5)
    for _ in range(50):
        NL, H = int(r.integers(1, 6)), int(r.integers(1, 9))
        L = int(r.choice([64, 256, 1024]))
        ret = float(r.uniform(0.2, 1.0))
        S = r.uniform(0, 1, (NL, H)).astype(np.float32)
        S[r.random((NL, H)) < 0.3] = 0.0
        kbar = math.floor(ret * L)
        if kbar < L and 4 + math.floor(0.5 * kbar) > kbar:
            continue
        b, _ = O.problem_budgets(_Prob(S, [L], [ret], pool=1))
        per = b.reshape(NL, H).sum(axis=1)
        assert (per == H * min(kbar, L)).all()
        if NL == 1:
            b0, _ = O.problem_budgets(_Prob(S, [L], [ret], pool=0))
            assert np.array_equal(b, b0)
