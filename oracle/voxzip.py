"""fp64 CPU oracle for decode-time decayed KV-cache eviction (VoxZip).

TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and bench.py's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library.  Plain numpy in fp64; every function is the definition written out.

Source: the VoxZip digest page ("VoxZip: Semantic-Anchored Temporal KV
Cache Compression for Long-Context Audio Inference"), method overview,
second stage "Temporally Decayed KV Cache Eviction" (its update equation and
concatenation rule), with the hyper-parameters of its details list:

  * every decode step t, per cache, the accumulated importance is
        A(t) = gamma * [A(t-1), 0] + softmax(q_t K_t^T / sqrt(d))
    where K_t is the cache including the new token's key, gamma = 0.95;
  * eviction keeps the first T = 4 tokens (attention sinks), the last M
    tokens with M equal to 20 % of the cache budget, and the N middle
    tokens of highest A(t); the new cache is the concatenation
    K[:T], K[I_hist], K[-M:] (V alike).

Readings taken where the page is open:
  * one cache per (sequence, layer, KV head); the G query heads of the KV
    head's group each give one softmax row over the cache, and A adds their
    mean (the plain GQA reading; a sum would select identically);
  * eviction runs when the cache holds more than its budget B rows, and
    brings it back to exactly B rows: M = floor(recent_frac * B),
    N = B - T - M;
  * A is trimmed with the same kept indices as K and V (the page leaves this
    open; gathering it is the reading that keeps A aligned with the cache);
  * I_hist lists the chosen middle positions in ascending order (the
    concatenation keeps temporal order); among equal A the lower position
    wins; -0.0 and +0.0 are equal.
"""
from __future__ import annotations

import math

import numpy as np


def attention_rows(q, k) -> np.ndarray:
    """q [G, d], k [n, d] -> p [G, n]: softmax over the n cached keys of
    q_g . k_j / sqrt(d), one row per query head (page: softmax(q_t K_t^T /
    sqrt(d)))."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    logits = (q @ k.T) / math.sqrt(q.shape[1])
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def accumulate(a_prev, q, k, gamma: float) -> np.ndarray:
    """A(t) = gamma * [A(t-1), 0] + mean over the G query heads of the
    softmax rows.  a_prev has n - 1 entries for a cache of n rows."""
    k = np.asarray(k, dtype=np.float64)
    n = k.shape[0]
    a_prev = np.asarray(a_prev, dtype=np.float64).reshape(-1)
    assert a_prev.shape[0] == n - 1
    padded = np.concatenate([a_prev, [0.0]])
    return gamma * padded + attention_rows(q, k).mean(axis=0)


def split(budget: int, n_sink: int, recent_frac: float):
    """(T, M, N) for a cache budget B: T sinks, M = floor(recent_frac * B)
    most recent tokens, N = B - T - M middle tokens."""
    M = int(math.floor(recent_frac * budget))
    N = budget - n_sink - M
    if N < 0:
        raise ValueError("budget smaller than sinks + recent window")
    return n_sink, M, N


def evict(A, budget: int, n_sink: int, recent_frac: float) -> np.ndarray:
    """Kept positions, ascending, for a cache of len(A) rows.

    No eviction (all positions) while the cache holds at most B rows;
    otherwise [0, T) + the N middle positions of largest A among [T, n - M)
    + [n - M, n)."""
    A = np.asarray(A, dtype=np.float64)
    n = A.shape[0]
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    T, M, N = split(budget, n_sink, recent_frac)
    mid = np.arange(T, n - M, dtype=np.int64)
    vals = A[mid] + 0.0                      # -0.0 -> +0.0
    order = np.lexsort((mid, -vals))         # A descending, then position
    chosen = np.sort(mid[order[:N]])
    return np.concatenate([np.arange(T, dtype=np.int64), chosen,
                           np.arange(n - M, n, dtype=np.int64)])


def step(q, k, v, a_prev, budget: int, gamma: float = 0.95, n_sink: int = 4,
         recent_frac: float = 0.2):
    """One decode step for one cache: -> dict(A (before eviction), kept,
    k_out, v_out, a_out)."""
    A = accumulate(a_prev, q, k, gamma)
    kept = evict(A, budget, n_sink, recent_frac)
    return dict(A=A, kept=kept, k_out=np.asarray(k)[kept], v_out=np.asarray(v)[kept],
                a_out=A[kept])
