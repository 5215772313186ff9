"""Pins for the WnW chunk-recall oracle (oracle/wnw.py).

WnW digest page, method section and reproduction notes: anchor attention
aggregated into 4 s / 2 s-stride chunk scores, top-3 chunks per step, release
after 3 unselected steps, per-segment static top-k for fixed heads.  The
pins are hand-worked cases, brute force on positions instead of blocks,
closed forms for uniform and one-hot attention, and invariants that a slip
(an off-by-one in the chunk range, the idle count, the slot order or the
quota rounding) breaks.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import oracle as O
from oracle import wnw as W


# -- geometry ---------------------------------------------------------------
@pytest.mark.parametrize("n,B,C", [(100, 4, 3), (101, 5, 4), (30, 2, 1), (20, 1, 1),
                                   (50, 2, 1), (51, 3, 2), (1, 1, 1)])
def test_chunk_counts_hand(n, B, C):
    assert W.n_blocks(n, 25) == B
    assert W.n_chunks(n, 25, 50) == C


@pytest.mark.parametrize("n", [1, 24, 25, 26, 49, 50, 51, 99, 100, 101, 1234])
@pytest.mark.parametrize("S,m", [(25, 2), (25, 1), (10, 3)])
def test_chunks_cover_every_position_and_start_every_stride(n, S, m):
    L = m * S
    C = W.n_chunks(n, S, L)
    cover = np.zeros(n, int)
    for c in range(C):
        lo, hi = W.chunk_range(c, n, S, L)
        assert lo == c * S and lo < n and hi - lo <= L
        cover[lo:hi] += 1
    assert cover.min() >= 1
    # no chunk could be dropped: the last one holds a position no other has
    lo, hi = W.chunk_range(C - 1, n, S, L)
    assert C == 1 or cover[hi - 1] == 1


# -- anchor attention and chunk scores --------------------------------------
def test_anchor_attention_matches_scipy_softmax():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((37, 16))
    want = softmax(q @ k.T / 4.0, axis=1).mean(axis=0)
    np.testing.assert_allclose(W.anchor_attention(q, k), want, rtol=1e-13)


def test_uniform_attention_gives_mass_proportional_to_chunk_length():
    n, S, L, A = 101, 25, 50, 3
    k = np.ones((n, 8))
    q = [np.random.default_rng(a).standard_normal((2, 8)) for a in range(A)]
    sigma = W.chunk_scores(q, [k] * A, n, S, L)
    want = [A * (min(c * S + L, n) - c * S) / n for c in range(W.n_chunks(n, S, L))]
    np.testing.assert_allclose(sigma, want, rtol=1e-13)
    assert sigma.tolist()[-1] < sigma.tolist()[0]   # the short last chunk (26 positions)


def test_one_hot_attention_selects_the_lower_chunk_holding_the_key():
    n, S, L = 200, 25, 50
    k = np.zeros((n, 8))
    k[130, 0] = 60.0                  # block 5; chunks 4 and 5 both hold it
    q = [np.eye(8)[:1]]
    sigma = W.chunk_scores(q, [k], n, S, L)
    assert math.isclose(sigma[4], sigma[5], rel_tol=1e-12) and sigma[4] > 0.99
    assert W.top_chunks(sigma, 1) == [4]
    assert W.top_chunks(sigma, 3)[:2] == [4, 5]


@pytest.mark.parametrize("n", [7, 50, 101, 333])
def test_chunk_scores_equal_position_sums(n):
    # brute force over positions, without blocks
    rng = np.random.default_rng(n)
    S, L = 25, 50
    qs = [rng.standard_normal((4, 16)) for _ in range(2)]
    ks = [rng.standard_normal((n, 16)) for _ in range(2)]
    sigma = W.chunk_scores(qs, ks, n, S, L)
    p = [softmax(q @ k.T / 4.0, axis=1).mean(axis=0) for q, k in zip(qs, ks)]
    for c in range(len(sigma)):
        want = sum(sum(pa[j] for j in range(c * S, min(c * S + L, n))) for pa in p)
        assert math.isclose(sigma[c], want, rel_tol=1e-12)


def test_top_chunks_ties_and_short_lists():
    assert W.top_chunks([1.0, 3.0, 3.0, 2.0], 3) == [1, 2, 3]
    assert W.top_chunks([0.5, 0.5], 3) == [0, 1]
    assert W.top_chunks([2.0], 3) == [0]


# -- residency ----------------------------------------------------------------
def test_release_after_three_unselected_steps_hand():
    st = W.Residency(n=500, stride=25, length=50, top=1, release_after=3)
    script = [5, 7, 7, 7, 5, 9, 9, 9, 9]
    # idle count of chunk 5 after each step (-1 = released)
    want5 = [0, 1, 2, -1, 0, 1, 2, -1, -1]
    for c, w in zip(script, want5):
        st, _ = W.update(st, [c])
        assert st.idle[5] == w


def test_slots_hand_case():
    # S = 25, m = 2, K = 1, H = 1: only the selected chunk stays; 2 slots
    st = W.Residency(n=200, stride=25, length=50, top=1, release_after=1)
    assert st.slot_cap() == 2
    st, rec = W.update(st, [3])        # blocks 3, 4 -> slots 0, 1
    assert rec == [(3, 0), (4, 1)]
    st, rec = W.update(st, [4])        # blocks 4, 5: 4 keeps slot 1, 3 frees slot 0
    assert rec == [(5, 0)] and st.slot_of_block[4] == 1 and st.slot_of_block[3] == -1
    st, rec = W.update(st, [4])        # nothing new
    assert rec == []
    st, rec = W.update(st, [0])        # blocks 0, 1 into slots 0, 1
    assert rec == [(0, 0), (1, 1)]
    assert st.block_of_slot == [0, 1]


def test_residency_invariants_on_a_random_walk():
    rng = np.random.default_rng(1)
    n, S, L, K, H = 3000, 25, 50, 3, 3
    st = W.Residency(n, S, L, K, H)
    C = W.n_chunks(n, S, L)
    for _ in range(200):
        sel = W.top_chunks(rng.random(C), K)
        prev = st
        st, rec = W.update(st, sel)
        res = st.resident_blocks()
        assert sum(z >= 0 for z in st.idle) <= K * H
        for c in sel:
            assert st.idle[c] == 0
        for b, s in enumerate(st.slot_of_block):
            assert (s >= 0) == res[b]
            if s >= 0:
                assert st.block_of_slot[s] == b
                if prev.slot_of_block[b] >= 0:
                    assert prev.slot_of_block[b] == s      # a kept block keeps its slot
        assert sorted(b for b, _ in rec) == [b for b, _ in rec]
        assert all(prev.slot_of_block[b] < 0 for b, _ in rec)


def test_recall_copies_rows_into_slots():
    n, S = 130, 25
    host = np.arange(n * 2, dtype=np.float64).reshape(n, 2)
    slots = np.full((4 * S, 2), -1.0)
    W.recall(slots, host, [(5, 2), (1, 0)], n, S)
    assert np.array_equal(slots[2 * S:2 * S + 5], host[125:130])
    assert np.all(slots[2 * S + 5:3 * S] == -1)
    assert np.array_equal(slots[0:S], host[25:50])


# -- fixed heads ----------------------------------------------------------------
def test_segment_quotas_hand():
    assert W.segment_quotas(13, 130, 50) == [5, 5, 3]
    # 10 * (50, 50, 30) / 130 = 3.85, 3.85, 2.31 -> floors 3, 3, 2, two more by remainder
    assert W.segment_quotas(10, 130, 50) == [4, 4, 2]
    assert W.segment_quotas(0, 130, 50) == [0, 0, 0]
    assert W.segment_quotas(130, 130, 50) == [50, 50, 30]


@pytest.mark.parametrize("k,ncand,seg", [(7, 1000, 50), (999, 1000, 50), (1, 77, 10),
                                         (500, 30000, 50), (3, 3, 64)])
def test_segment_quotas_sum_and_bounds(k, ncand, seg):
    q = W.segment_quotas(k, ncand, seg)
    assert sum(q) == k
    for j, qj in enumerate(q):
        ln = min(seg, ncand - j * seg)
        assert k * ln // ncand <= qj <= -(-k * ln // ncand) and qj <= ln


def test_one_segment_is_the_global_top_k():
    rng = np.random.default_rng(2)
    L, w = 300, 32
    s = np.round(rng.random(L), 2)
    for b in (w, w + 1, 100, L):
        assert np.array_equal(W.segment_select(s, w, b, L), O.select(s, w, b))


def test_unit_segments_keep_the_first_positions():
    # every segment has one position and the same remainder: the k lowest win
    s = np.random.default_rng(3).random(100)
    got = W.segment_select(s, 10, 10 + 7, 1)
    assert got.tolist() == list(range(7)) + list(range(90, 100))


def test_segment_select_hand():
    s = np.array([0.1, 0.9, 0.5, -0.0, 0.0, 0.3, 0.8, 0.8, 0.2, 0.4, 7.0, 7.0])
    # w = 2, candidates 0..9 in segments of 4: (0..3), (4..7), (8..9); k = 5
    # quotas 5 * (4, 4, 2) / 10 = 2, 2, 1
    got = W.segment_select(s, 2, 7, 4)
    assert got.tolist() == [1, 2, 6, 7, 9, 10, 11]
    # signed zeros tie: lower position first
    got = W.segment_select(np.array([-0.0, 0.0, -1.0, 5.0, 5.0]), 2, 3, 3)
    assert got.tolist() == [0, 3, 4]
