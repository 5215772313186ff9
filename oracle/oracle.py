"""Python face of the fp64 CPU oracle (test infrastructure only).

Only tests/, the smoke check and bench.py's CPU-baseline leg may import this
module.  It loads ``libkvc_oracle.so`` (plain C, built from kvc_oracle.c by
``oracle/build.py``) and adds the per-unit driver: bf16/fp32 widening to
fp64, the GQA grouping of window queries, the segment layout of the compacted
cache, and a thread pool over units (one C call per unit; ctypes releases the
GIL while the C code runs).

Each step follows the page passage cited in kvc_oracle.c; gathering is a
numpy fancy-index copy of whole rows.
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes
import os
import pathlib
import threading

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_LIB_PATH = _HERE / "libkvc_oracle.so"
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)
_fp = ctypes.POINTER(ctypes.c_float)


class OracleError(RuntimeError):
    pass


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not _LIB_PATH.exists():
                from oracle import build as _b
                _b.build()
            L = ctypes.CDLL(str(_LIB_PATH))
            L.kvo_scores.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
            L.kvo_dft.argtypes = [ctypes.c_int, _dp, _dp, _dp]
            L.kvo_sss.argtypes = [ctypes.c_int, _dp, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_int, _dp, _ip, _dp, _dp]
            L.kvo_budget.argtypes = [ctypes.c_int, _fp, ctypes.c_int, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_int, _ip]
            L.kvo_select.argtypes = [ctypes.c_int, _dp, ctypes.c_int, ctypes.c_int, _ip]
            for f in (L.kvo_scores, L.kvo_dft, L.kvo_sss, L.kvo_budget, L.kvo_select):
                f.restype = ctypes.c_int
            _lib = L
    return _lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def widen(x, dtype: str) -> np.ndarray:
    """Exact widening of stored inputs to fp64 (bf16 bits are uint16)."""
    if dtype == "bf16":
        a = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return a.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Single-step wrappers
# --------------------------------------------------------------------------
def scores(q, k) -> np.ndarray:
    """q [gw, d], k [L, d] (float) -> s [L] fp64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    gw, d = q.shape
    L = k.shape[0]
    assert k.shape[1] == d
    s = np.empty(L, dtype=np.float64)
    _check(lib().kvo_scores(gw, L, d, _ptr(q, _dp), _ptr(k, _dp), _ptr(s, _dp)), "scores")
    return s


def scores_maxpool(q, k, W: int) -> np.ndarray:
    """Max over query heads of each head's mean softmax row: q [G*W, d]
    holds the heads' W window queries head after head; each head's row is
    the mean-pooled score of its own W queries (kvo_scores on them)."""
    q = np.asarray(q, dtype=np.float64)
    G = q.shape[0] // W
    assert G * W == q.shape[0]
    return np.max(np.stack([scores(q[g * W:(g + 1) * W], k) for g in range(G)]), axis=0)


def dft(s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float64)
    L = s.shape[0]
    re = np.empty(L // 2 + 1)
    im = np.empty(L // 2 + 1)
    _check(lib().kvo_dft(L, _ptr(s, _dp), _ptr(re, _dp), _ptr(im, _dp)), "dft")
    return re + 1j * im


def sss(s, alpha: float, rho: float, kstar: int | None = None):
    """-> (s_hat [L], kstar, energy [L//2+1], lowpass [L])."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    L = s.shape[0]
    sh = np.empty(L)
    lp = np.empty(L)
    E = np.empty(L // 2 + 1)
    ks = ctypes.c_int(0)
    _check(lib().kvo_sss(L, _ptr(s, _dp), float(alpha), float(rho),
                         -1 if kstar is None else int(kstar),
                         _ptr(sh, _dp), ctypes.byref(ks), _ptr(E, _dp), _ptr(lp, _dp)), "sss")
    return sh, int(ks.value), E, lp


def budget(S, L: int, retention: float, base_ratio: float = 0.5, window: int = 32) -> np.ndarray:
    S = np.ascontiguousarray(np.ravel(S), dtype=np.float32)
    b = np.empty(S.shape[0], dtype=np.int32)
    _check(lib().kvo_budget(S.shape[0], _ptr(S, _fp), int(L), float(retention),
                            float(base_ratio), int(window), _ptr(b, _ip)), "budget")
    return b


def budget_rc(S, L, retention, base_ratio=0.5, window=32) -> int:
    S = np.ascontiguousarray(np.ravel(S), dtype=np.float32)
    b = np.empty(max(1, S.shape[0]), dtype=np.int32)
    return int(lib().kvo_budget(S.shape[0], _ptr(S, _fp), int(L), float(retention),
                                float(base_ratio), int(window), _ptr(b, _ip)))


def select(s_hat, window: int, b: int) -> np.ndarray:
    s_hat = np.ascontiguousarray(s_hat, dtype=np.float64)
    kept = np.empty(max(1, int(b)), dtype=np.int32)
    _check(lib().kvo_select(s_hat.shape[0], _ptr(s_hat, _dp), int(window), int(b),
                            _ptr(kept, _ip)), "select")
    return kept[:int(b)]


def gather(x, kept) -> np.ndarray:
    return np.asarray(x)[np.asarray(kept, dtype=np.int64)]


# --------------------------------------------------------------------------
# Whole-problem driver
# --------------------------------------------------------------------------
def unit_compress(qu, ku, dtype: str, b: int, alpha: float, rho: float, window: int,
                  score_pool: int = 0):
    """One (sequence, layer, KV head) unit: scores -> SSS -> top-k.

    qu: [G, W, d] stored window queries of the KV head's group; ku: [L, d].
    score_pool 1 takes the max over the G heads of the head means.
    Returns dict(s, s_hat, kstar, energy, kept).
    """
    q = widen(qu, dtype).reshape(-1, np.asarray(qu).shape[-1])
    k = widen(ku, dtype)
    s = scores_maxpool(q, k, np.asarray(qu).shape[1]) if score_pool == 1 else scores(q, k)
    s_hat, ks, E, _ = sss(s, alpha, rho)
    kept = select(s_hat, window, b)
    return dict(s=s, s_hat=s_hat, kstar=ks, energy=E, kept=kept)


def problem_budgets(prob, budget_pool=None):
    """Budgets for every unit in (seq, layer, head) order, plus offsets.

    budget_pool 0 (default of the config): one pool per sequence over all its
    (layer, KV head) heads; 1: the same budget rule applied to each layer's
    KV heads on their own."""
    cfg, hdr = prob.cfg, prob.hdr
    pool = cfg.budget_pool if budget_pool is None else budget_pool
    S = np.asarray(hdr.head_scores).reshape(cfg.n_layers, cfg.n_kv_heads)
    out = []
    for i in range(cfg.n_seq):
        L, r = int(hdr.lengths[i]), float(hdr.retention[i])
        if pool == 1:
            for l in range(cfg.n_layers):
                out.append(budget(S[l], L, r, cfg.base_ratio, cfg.window))
        else:
            out.append(budget(S, L, r, cfg.base_ratio, cfg.window))
    b = np.concatenate(out).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(b, dtype=np.int64)]).astype(np.int64)
    return b, off


def unit_index(cfg, i, l, h):
    return (i * cfg.n_layers + l) * cfg.n_kv_heads + h


def unit_inputs(prob, i, l, h):
    cfg, hdr = prob.cfg, prob.hdr
    G = cfg.gqa
    st = hdr.seq_start
    qu = prob.q[i, l, h * G:(h + 1) * G]
    ku = prob.k[l, h, st[i]:st[i + 1]]
    vu = prob.v[l, h, st[i]:st[i + 1]]
    return qu, ku, vu


def threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def compress(prob, units=None, n_threads=None):
    """Oracle for a whole Problem (or the listed units (i, l, h)).

    Returns dict(budgets, offsets, units={(i,l,h): unit result with k_out,
    v_out, idx}).
    """
    cfg = prob.cfg
    b, off = problem_budgets(prob)
    if units is None:
        units = [(i, l, h) for i in range(cfg.n_seq) for l in range(cfg.n_layers)
                 for h in range(cfg.n_kv_heads)]

    def run(key):
        i, l, h = key
        qu, ku, vu = unit_inputs(prob, i, l, h)
        u = unit_index(cfg, i, l, h)
        r = unit_compress(qu, ku, cfg.dtype, int(b[u]), cfg.alpha, cfg.rho, cfg.window,
                          cfg.score_pool)
        r["k_out"] = gather(ku, r["kept"])
        r["v_out"] = gather(vu, r["kept"])
        r["idx"] = r["kept"]
        return key, r

    n = n_threads or threads()
    with _cf.ThreadPoolExecutor(max(1, n)) as ex:
        res = dict(ex.map(run, units))
    return dict(budgets=b, offsets=off, units=res)
