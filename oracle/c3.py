"""CPU oracle for C3 speech-guided KV retrieval.

TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and bench.py's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library.  Plain numpy; every function follows the C3 digest page ("C3:
Speech-Guided KV Retrieval for Long-Context SpeechLLM Inference"): the
overall flow (tree at prefill, per-step node scoring, budget fill and
gather), shared competition within a KV head's group (the max-cosine score
equation), content clustering (recursive bisecting k-means per layer and KV
head, an initial frontier of mean node size 16, node sizes down to 4),
adaptive resolution (the EMA equation, R paired split/merge exchanges per
step, children inheriting the parent's state, a merged parent taking the max
of its children, candidates found by masked max/min reductions) and the
reproduction notes (8 k-means iterations, seed 0, lambda = 0.5, R = 2,
retrieval bypassed when the audio fits the budget).

The tree is a set of integer decisions taken by floating point, so every
decision is defined here in the precision and operation order a GPU can
reproduce exactly (readings of the page):
  * one index per (sequence, layer, KV head) cache of n audio keys (bf16);
    keys must be finite with |k| < 4096 and n <= 2^17;
  * the keys are first snapped to the grid 2^-24 (only |k| < 2^-17 moves),
    so every sum of them below is exact in fp64 and the same in any order;
  * a node with more than LEAF = 4 keys splits by 8 Lloyd iterations of
    2-means; depth is capped at MAX_DEPTH = 24;
  * assignment: w = mu1 - mu0 rounded to fp32 and then to 16 significant
    bits (|w| < 2^-100 -> 0), m = (mu0 + mu1) / 2 rounded to fp32,
    b = sum_c w_c m_c and s(k) = sum_c k_c w_c in fp32, both summed in
    column order (each product rounded to fp32, then added to the running
    sum); the key joins cluster 1 iff s(k) > b (the nearest-centroid test
    written as the side of the bisecting hyperplane; a key on it joins
    cluster 0).  Every k_c w_c is exact in fp32, so a fused multiply-add
    gives the same s(k);
  * a split that leaves a cluster empty at any iteration is abandoned (the
    node stays a leaf); a mean is the exact member sum divided by the
    count, correctly rounded in fp64 (the plain definition of the mean);
  * "seed 0": the initial centroids are two distinct member keys chosen by
    the SplitMix64 mixing function (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014) of (seed, cache, depth,
    start, size);
  * members keep their relative order; cluster 0 is the left child; nodes
    are numbered breadth first, children in parent order, left first, so
    within one depth ids follow the first member's place ("start");
  * the stored centroid of a node is its exact mean rounded to fp32 and then
    to bf16 (round to nearest even both times);
  * the initial frontier is every node at depth round(log2(n / 16)) plus
    the leaves above it, listed by start (the frontier tiles the member
    order, so start orders it);
  * sigma_n = max_g cos(q_g, c_n) (0 where a norm is 0); nodes are ranked by
    sigma descending, ties by start; whole nodes are taken until B keys, the
    node that crosses B gives the first members of its range of the member
    order; kept positions are listed ascending; n <= B keeps everything and
    leaves the frontier state unchanged;
  * after the step, e = lambda e + (1 - lambda) sigma (fp64, e starts at 0);
    the split candidates are the R frontier nodes with children of highest
    e (ties by start); the merge candidates are the R sibling pairs on the
    frontier, neither of them a split candidate, of lowest max(e_left,
    e_right) (ties by start); the first min(#splits, #merges) of each are
    applied.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

LEAF = 4
ITERS = 8
MAX_DEPTH = 24
GRANULARITY = 16
GRID = 2.0 ** -24
KEY_LIMIT = 4096.0
N_LIMIT = 1 << 17
W_FLUSH = 2.0 ** -100
MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# helpers of the decisions
# ---------------------------------------------------------------------------
def splitmix64(x: int) -> int:
    """One SplitMix64 output for state x: add the golden gamma, then two
    xor-shift-multiply rounds and a final xor-shift."""
    z = (x + 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def init_pair(seed: int, cache: int, depth: int, start: int, size: int):
    """Two distinct member indices in [0, size) for a node's initial
    centroids."""
    h0 = splitmix64((seed ^ (cache << 40) ^ (depth << 32) ^ start) & MASK64)
    h1 = splitmix64(h0)
    a0 = h0 % size
    a1 = (a0 + 1 + h1 % (size - 1)) % size
    return int(a0), int(a1)


def quantize(K) -> np.ndarray:
    """Keys snapped to the 2^-24 grid (exact in fp64)."""
    K = np.asarray(K, dtype=np.float64)
    return np.rint(K / GRID) * GRID


def round16(x32) -> np.ndarray:
    """fp32 values rounded to 16 significant bits (nearest, ties to even)."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7F + ((b >> 8) & 1)) & 0xFFFFFF00
    return r.astype(np.uint32).view(np.float32)


def to_bf16(x64) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (nearest even both times); returned as fp32."""
    b = np.ascontiguousarray(np.asarray(x64, dtype=np.float64).astype(np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bisector(mu0, mu1):
    """(w, b) of the hyperplane between two fp64 centroids (rows: nodes)."""
    mu0 = np.asarray(mu0, dtype=np.float64)
    mu1 = np.asarray(mu1, dtype=np.float64)
    w = round16((mu1 - mu0).astype(np.float32))
    w = np.where(np.abs(w) < W_FLUSH, np.float32(0), w).astype(np.float32)
    m = (0.5 * (mu0 + mu1)).astype(np.float32)
    b = np.zeros(w.shape[:-1], dtype=np.float32)
    for c in range(w.shape[-1]):                     # column order, fp32
        b = b + w[..., c] * m[..., c]
    return w, b


def assign(X32, W, b) -> np.ndarray:
    """to1[j] = s(X_j) > b_j with s summed in fp32 in column order; W and b
    are per row (the row's node)."""
    acc = np.zeros(X32.shape[0], dtype=np.float32)
    for c in range(X32.shape[1]):
        acc = acc + X32[:, c] * W[:, c]
    return acc > b


# ---------------------------------------------------------------------------
# tree
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Tree:
    start: np.ndarray     # int64 [nodes]: first member's place in perm
    size: np.ndarray      # int64 [nodes]
    left: np.ndarray      # int64 [nodes]: left child id or -1 (right = left + 1)
    parent: np.ndarray    # int64 [nodes]: -1 for the root
    depth: np.ndarray     # int64 [nodes]
    centroid: np.ndarray  # float32 [nodes, d], values of bf16
    perm: np.ndarray      # int64 [n]: members of x are perm[start:start+size]

    @property
    def n_nodes(self) -> int:
        return int(self.start.shape[0])


def check_keys(K) -> None:
    K = np.asarray(K, dtype=np.float64)
    if K.shape[0] > N_LIMIT:
        raise ValueError("more than 2^17 keys in one cache")
    if not np.isfinite(K).all() or (np.abs(K) >= KEY_LIMIT).any():
        raise ValueError("keys must be finite with |k| < 4096")


def _level_two_means(Xq, seg, sizes, a0, a1):
    """8 Lloyd iterations for every node of one level side by side.  The
    nodes are independent and each follows its own sequence exactly; running
    them together only batches the array operations.  Xq: members of all
    nodes (grouped by node, member order), seg: node of each row."""
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    X32 = Xq.astype(np.float32)                      # exact: bf16 values
    mu0 = Xq[offs + a0].copy()
    mu1 = Xq[offs + a1].copy()
    alive = np.ones(len(sizes), dtype=bool)
    S = np.add.reduceat(Xq, offs, axis=0)            # exact sums
    to1 = np.zeros(len(seg), dtype=bool)
    with np.errstate(invalid="ignore", divide="ignore"):
        for _ in range(ITERS):
            w, b = bisector(mu0, mu1)
            t = assign(X32, w[seg], b[seg])
            to1 = np.where(alive[seg], t, to1)
            n1 = np.bincount(seg, weights=to1, minlength=len(sizes)).astype(np.int64)
            alive &= (n1 > 0) & (n1 < sizes)
            S1 = np.add.reduceat(Xq * to1[:, None], offs, axis=0)
            mu1 = np.where(alive[:, None], S1 / n1[:, None], mu1)
            mu0 = np.where(alive[:, None], (S - S1) / (sizes - n1)[:, None], mu0)
    return alive, to1, mu0, mu1


def build_tree(K, cache: int = 0, seed: int = 0) -> Tree:
    """Recursive bisecting 2-means over the rows of K (values of bf16 keys),
    level by level."""
    check_keys(K)
    Kq = quantize(K)
    n, d = Kq.shape
    perm = np.arange(n, dtype=np.int64)
    if n == 0:
        z = np.zeros(0, np.int64)
        return Tree(z, z, z, z, z, np.zeros((0, d), np.float32), perm)
    start, size, left, parent, depth = [0], [n], [-1], [-1], [0]
    means = [Kq.sum(axis=0) / n]
    lo, hi = 0, 1
    for dep in range(MAX_DEPTH):
        cand = [x for x in range(lo, hi) if size[x] > LEAF]
        if not cand:
            break
        sizes = np.array([size[x] for x in cand], dtype=np.int64)
        pos = np.concatenate([np.arange(start[x], start[x] + size[x]) for x in cand])
        seg = np.repeat(np.arange(len(cand)), sizes)
        pairs = [init_pair(seed, cache, dep, start[x], size[x]) for x in cand]
        a0 = np.array([p[0] for p in pairs], dtype=np.int64)
        a1 = np.array([p[1] for p in pairs], dtype=np.int64)
        alive, to1, mu0, mu1 = _level_two_means(Kq[perm[pos]], seg, sizes, a0, a1)
        newperm = perm.copy()
        base = 0
        for i, x in enumerate(cand):
            m = int(sizes[i])
            rows = slice(base, base + m)
            base += m
            if not alive[i]:
                continue
            s = start[x]
            idx = perm[s:s + m]
            t = to1[rows]
            n0 = int((~t).sum())
            newperm[s:s + m] = np.concatenate([idx[~t], idx[t]])
            left[x] = len(start)
            for cs, cm, mu in ((s, n0, mu0[i]), (s + n0, m - n0, mu1[i])):
                start.append(cs)
                size.append(cm)
                left.append(-1)
                parent.append(x)
                depth.append(dep + 1)
                means.append(mu)
        perm = newperm
        lo, hi = hi, len(start)
    return Tree(np.array(start, np.int64), np.array(size, np.int64), np.array(left, np.int64),
                np.array(parent, np.int64), np.array(depth, np.int64),
                to_bf16(np.array(means)), perm)


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
def frontier_depth(n: int) -> int:
    """round(log2(n / 16)), at least 0."""
    if n <= 0:
        return 0
    return max(0, int(round(math.log2(n / GRANULARITY))))


def initial_frontier(tree: Tree, n: int) -> np.ndarray:
    """Frontier node ids, listed by start."""
    D0 = frontier_depth(n)
    on = (tree.depth == D0) | ((tree.left < 0) & (tree.depth < D0))
    ids = np.nonzero(on)[0]
    return ids[np.argsort(tree.start[ids], kind="stable")]


def node_scores(tree: Tree, F, q) -> np.ndarray:
    """sigma per frontier entry: max over the group's query heads of the
    cosine of query and centroid (fp64; 0 where a norm is 0)."""
    q = np.asarray(q, dtype=np.float64)
    C = tree.centroid[np.asarray(F, dtype=np.int64)].astype(np.float64)
    cn = np.sqrt((C * C).sum(axis=1))
    qn = np.sqrt((q * q).sum(axis=1))
    dots = C @ q.T                                   # [A, G]
    den = cn[:, None] * qn[None, :]
    cos = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
    return cos.max(axis=1)


def retrieve(tree: Tree, F, sig, n: int, B: int) -> np.ndarray:
    """Kept positions (ascending): frontier nodes by sigma descending, ties
    by start; whole nodes until B keys, the crossing node gives its first
    members; everything when n <= B."""
    if n <= B:
        return np.arange(n, dtype=np.int64)
    F = np.asarray(F, dtype=np.int64)
    sig = np.asarray(sig, dtype=np.float64)
    order = np.lexsort((tree.start[F], -sig))
    kept, room = [], B
    for i in order:
        if room == 0:
            break
        x = F[i]
        s, m = int(tree.start[x]), int(tree.size[x])
        take = min(m, room)
        kept.append(tree.perm[s:s + take])
        room -= take
    return np.sort(np.concatenate(kept))


def update_frontier(tree: Tree, F, e, sig, lam: float = 0.5, R: int = 2):
    """EMA of the entries' scores, then up to R split/merge exchanges.
    F: ids listed by start, e: state per entry.  Returns (F', e')."""
    F = np.asarray(F, dtype=np.int64)
    A = len(F)
    e = lam * np.asarray(e, dtype=np.float64) + (1.0 - lam) * np.asarray(sig, dtype=np.float64)
    # R masked max reductions over the nodes with children
    can_split = tree.left[F] >= 0
    splits = []
    for _ in range(R):
        best = -1
        for i in range(A):
            if can_split[i] and i not in splits and (best < 0 or e[i] > e[best]):
                best = i
        if best < 0:
            break
        splits.append(best)
    # sibling pairs on the frontier are adjacent entries (i, i+1)
    pair_ok = np.zeros(A, dtype=bool)
    for i in range(A - 1):
        p = tree.parent[F[i]]
        if p >= 0 and tree.left[p] == F[i] and F[i + 1] == F[i] + 1 \
                and i not in splits and (i + 1) not in splits:
            pair_ok[i] = True
    pri = np.full(A, np.inf)
    pri[:-1] = np.maximum(e[:-1], e[1:]) if A > 1 else pri[:-1]
    merges = []
    for _ in range(R):
        best = -1
        for i in range(A):
            if pair_ok[i] and i not in merges and (best < 0 or pri[i] < pri[best]):
                best = i
        if best < 0:
            break
        merges.append(best)
    k = min(len(splits), len(merges))
    split_set, merge_set = set(splits[:k]), set(merges[:k])
    F2, e2 = [], []
    i = 0
    while i < A:
        if i in split_set:
            l = int(tree.left[F[i]])
            F2 += [l, l + 1]
            e2 += [e[i], e[i]]
            i += 1
        elif i in merge_set:
            F2.append(int(tree.parent[F[i]]))
            e2.append(max(e[i], e[i + 1]))
            i += 2
        else:
            F2.append(int(F[i]))
            e2.append(e[i])
            i += 1
    return np.array(F2, dtype=np.int64), np.array(e2, dtype=np.float64)


def step(tree: Tree, F, e, q, n: int, B: int, lam: float = 0.5, R: int = 2, sig=None):
    """One decode step for one cache -> dict(sigma, kept, F, e).  sigma may
    be given (scores taken elsewhere); a cache that fits the budget bypasses
    retrieval and keeps its frontier state."""
    F = np.asarray(F, dtype=np.int64)
    if n <= B:
        return dict(sigma=None, kept=np.arange(n, dtype=np.int64), F=F.copy(),
                    e=np.asarray(e, dtype=np.float64).copy())
    if sig is None:
        sig = node_scores(tree, F, q)
    kept = retrieve(tree, F, sig, n, B)
    F2, e2 = update_frontier(tree, F, e, sig, lam, R)
    return dict(sigma=sig, kept=kept, F=F2, e=e2)
