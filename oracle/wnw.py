"""fp64 CPU oracle for decode-time chunk recall (WnW).

TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and bench.py's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library.  Plain numpy in fp64 and Python integers; every function is the
definition written out.

Source: the WnW digest page ("WnW: Waxing-and-Waning KV Cache for Long-Form
Speech LLMs"): its summary and method sections on the three head roles, and
its reproduction notes:

  * anchor KV heads keep their whole audio KV on the GPU; every decode step
    their attention over the audio positions is aggregated into importance
    scores of time chunks;
  * tidal KV heads keep a full copy on the host; the GPU holds only the
    chunks currently recalled; the audio is cut into 4 s chunks with a 2 s
    stride, the 3 best chunks are selected every step, and a chunk leaves the
    GPU only after 3 consecutive steps without being selected (the host copy
    stays, so it can be recalled again);
  * fixed KV heads keep only a static subset chosen at prefill segment by
    segment (instead of one top-k over the whole audio), so that no stretch
    of a long recording is left without cache.

Readings taken where the page is open:
  * chunk geometry in tokens: stride S (2 s) and length W = m S (4 s, m = 2);
    block b = positions [b S, min((b + 1) S, n)), B = ceil(n / S) blocks;
    chunk c = blocks c .. c + m - 1 (clipped), C = max(1, B - m + 1) chunks,
    so the chunks start every S tokens and together cover all n positions;
  * an anchor's attention over the audio is the mean over its G query heads
    of softmax(q_g k_j / sqrt(d)) over the n audio keys; a chunk's score is
    the attention mass on its positions, summed over the anchor heads;
  * top-K chunks by score, ties to the lower chunk index;
  * residency per chunk: selected -> resident with idle count 0; a resident
    chunk not selected counts one more idle step and is released when the
    count reaches H (= 3); one residency per sequence, shared by all of its
    tidal heads (the scores come from the shared anchors);
  * storage of recalled KV in blocks of S rows (overlapping chunks share
    blocks): a block is resident while any resident chunk covers it; each
    tidal head has a slot buffer of K * H * m blocks (the most that can be
    resident); a block that stays resident keeps its slot, released blocks
    free theirs, and newly resident blocks, in ascending block order, take
    the free slots in ascending slot order;
  * fixed heads: the candidates [0, L - w) are cut into segments of `seg`
    positions (last one shorter); the k = b - w kept candidates are shared
    among segments in proportion to their lengths by largest remainder
    (ties to the lower segment); each segment keeps its quota of largest
    s_hat (ties to the lower position, -0.0 == +0.0); kept positions in
    ascending order, then the local window [L - w, L).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

FIXED, ANCHOR, TIDAL = 0, 1, 2


# ---------------------------------------------------------------------------
# Chunk geometry
# ---------------------------------------------------------------------------
def n_blocks(n: int, stride: int) -> int:
    return -(-n // stride)


def n_chunks(n: int, stride: int, length: int) -> int:
    m = length // stride
    return max(1, n_blocks(n, stride) - m + 1)


def block_range(b: int, n: int, stride: int):
    return b * stride, min((b + 1) * stride, n)


def chunk_range(c: int, n: int, stride: int, length: int):
    """Positions [c S, min(c S + W, n)) of chunk c."""
    return c * stride, min(c * stride + length, n)


# ---------------------------------------------------------------------------
# Anchor attention and chunk scores
# ---------------------------------------------------------------------------
def anchor_attention(q, k) -> np.ndarray:
    """q [G, d], k [n, d] -> p [n]: mean over the G query heads of the
    softmax over the n audio keys of q_g . k_j / sqrt(d)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    logits = (q @ k.T) / math.sqrt(q.shape[1])
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return (e / e.sum(axis=1, keepdims=True)).mean(axis=0)


def block_mass(p_anchors, n: int, stride: int) -> np.ndarray:
    """Sum over anchors of the attention mass on each block."""
    B = n_blocks(n, stride)
    out = np.zeros(B)
    for p in p_anchors:
        for b in range(B):
            lo, hi = block_range(b, n, stride)
            out[b] += float(np.sum(p[lo:hi]))
    return out


def chunk_scores_from_blocks(beta, n: int, stride: int, length: int) -> np.ndarray:
    m = length // stride
    B = len(beta)
    C = n_chunks(n, stride, length)
    return np.array([sum(beta[b] for b in range(c, min(c + m, B))) for c in range(C)])


def chunk_scores(q_anchors, k_anchors, n: int, stride: int, length: int) -> np.ndarray:
    """sigma_c = sum over anchors a of sum_{j in chunk c} p_a[j]."""
    p = [anchor_attention(q, k[:n]) for q, k in zip(q_anchors, k_anchors)]
    return chunk_scores_from_blocks(block_mass(p, n, stride), n, stride, length)


def top_chunks(sigma, K: int) -> list[int]:
    """The min(K, C) chunks of largest score, ties to the lower index, in
    that order (score descending, then index ascending)."""
    order = sorted(range(len(sigma)), key=lambda c: (-float(sigma[c]), c))
    return order[:min(K, len(sigma))]


# ---------------------------------------------------------------------------
# Residency and slots (one sequence)
# ---------------------------------------------------------------------------
@dataclass
class Residency:
    n: int
    stride: int
    length: int
    top: int = 3
    release_after: int = 3
    idle: list = field(default_factory=list)         # per chunk: -1 or 0..H-1
    slot_of_block: list = field(default_factory=list)
    block_of_slot: list = field(default_factory=list)

    def __post_init__(self):
        C = n_chunks(self.n, self.stride, self.length)
        B = n_blocks(self.n, self.stride)
        if not self.idle:
            self.idle = [-1] * C
            self.slot_of_block = [-1] * B
            self.block_of_slot = [-1] * self.slot_cap()

    def slot_cap(self) -> int:
        m = self.length // self.stride
        return min(n_blocks(self.n, self.stride), self.top * self.release_after * m)

    def resident_blocks(self) -> list[bool]:
        m = self.length // self.stride
        B = n_blocks(self.n, self.stride)
        res = [False] * B
        for c, z in enumerate(self.idle):
            if z >= 0:
                for b in range(c, min(c + m, B)):
                    res[b] = True
        return res

    def copy(self) -> "Residency":
        return Residency(self.n, self.stride, self.length, self.top, self.release_after,
                         list(self.idle), list(self.slot_of_block), list(self.block_of_slot))


def update(state: Residency, selected) -> tuple[Residency, list[tuple[int, int]]]:
    """One step: idle counts, residency, slots.  Returns the new state and
    the (block, slot) pairs recalled this step, by ascending block."""
    s = state.copy()
    sel = set(selected)
    for c in range(len(s.idle)):
        if c in sel:
            s.idle[c] = 0
        elif s.idle[c] >= 0:
            s.idle[c] += 1
            if s.idle[c] >= s.release_after:
                s.idle[c] = -1
    res = s.resident_blocks()
    for b, slot in enumerate(s.slot_of_block):
        if slot >= 0 and not res[b]:
            s.block_of_slot[slot] = -1
            s.slot_of_block[b] = -1
    free = [i for i, b in enumerate(s.block_of_slot) if b < 0]
    new = [b for b in range(len(res)) if res[b] and s.slot_of_block[b] < 0]
    assert len(new) <= len(free)
    recalled = []
    for b, slot in zip(new, free):
        s.slot_of_block[b] = slot
        s.block_of_slot[slot] = b
        recalled.append((b, slot))
    return s, recalled


def recall(slot_rows, host_rows, recalled, n: int, stride: int):
    """Copy each recalled block's rows of one tidal head from its host copy
    [n, d] into its slot of the slot buffer [slots * stride, d]."""
    for b, slot in recalled:
        lo, hi = block_range(b, n, stride)
        slot_rows[slot * stride: slot * stride + (hi - lo)] = host_rows[lo:hi]


def step(state: Residency, q_anchors, k_anchors):
    """Scores, top-K, residency update: -> (sigma, selected, state, recalled)."""
    sigma = chunk_scores(q_anchors, k_anchors, state.n, state.stride, state.length)
    sel = top_chunks(sigma, state.top)
    new_state, recalled = update(state, sel)
    return sigma, sel, new_state, recalled


# ---------------------------------------------------------------------------
# Fixed heads: segment-wise static top-k at prefill
# ---------------------------------------------------------------------------
def segment_quotas(k: int, ncand: int, seg: int) -> list[int]:
    """Share k kept positions among the segments of [0, ncand) in proportion
    to their lengths, largest remainder, ties to the lower segment."""
    J = -(-ncand // seg) if ncand > 0 else 0
    lens = [min(seg, ncand - j * seg) for j in range(J)]
    fl = [k * ln // ncand for ln in lens]
    rem = [k * ln % ncand for ln in lens]
    R = k - sum(fl)
    order = sorted(range(J), key=lambda j: (-rem[j], j))
    for j in order[:R]:
        fl[j] += 1
    return fl


def segment_select(s_hat, window: int, b: int, seg: int) -> np.ndarray:
    s = np.asarray(s_hat, dtype=np.float64)
    L = s.shape[0]
    ncand = L - window
    k = b - window
    assert 0 <= k <= ncand
    kept = []
    if ncand > 0:
        q = segment_quotas(k, ncand, seg)
        for j, qj in enumerate(q):
            lo, hi = j * seg, min((j + 1) * seg, ncand)
            vals = [0.0 if s[p] == 0.0 else float(s[p]) for p in range(lo, hi)]
            order = sorted(range(lo, hi), key=lambda p: (-vals[p - lo], p))
            kept.extend(sorted(order[:qj]))
    kept.extend(range(ncand, L))
    return np.array(kept, dtype=np.int32)
