"""ctypes binding of libkvc.so (the C ABI declared in include/kvc.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  torch is imported before the library is loaded so that the
process has a single HIP runtime (torch's), which libkvc.so then binds to.
"""
from __future__ import annotations

import ctypes
import pathlib
import threading

import torch  # noqa: F401  (loads the HIP runtime libkvc.so binds to)

_PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = _PKG / "libkvc.so"

KVC_OK = 0
KVC_ERR_INVALID_ARG = 1
KVC_ERR_UNSUPPORTED = 2
KVC_ERR_BUDGET = 3
KVC_ERR_WORKSPACE = 4
KVC_ERR_HIP = 5
KVC_BF16 = 0
KVC_F32 = 1

EXPORTS = ("kvc_plan", "kvc_compress", "kvc_compress_layers", "kvc_scores", "kvc_score_stats",
           "kvc_score_pool", "kvc_smooth", "kvc_budget", "kvc_select", "kvc_gather",
           "kvc_compress_noalloc", "kvc_status_str", "kvc_last_hip_error")
# workspace limit of kvc_compress_noalloc (KVC_NOALLOC_MAX_WORKSPACE)
KVC_NOALLOC_MAX_WORKSPACE = 64 << 20
# include/kvc_voxzip.h
VZ_EXPORTS = ("kvc_vz_plan", "kvc_vz_step", "kvc_vz_accumulate", "kvc_vz_evict",
              "kvc_vz_gather", "kvc_vz_step_inplace")
# include/kvc_c3.h
C3_EXPORTS = ("kvc_c3_plan", "kvc_c3_build", "kvc_c3_step", "kvc_c3_score", "kvc_c3_select",
              "kvc_c3_update", "kvc_c3_gather")
# include/kvc_wnw.h
WNW_EXPORTS = ("kvc_wnw_plan", "kvc_wnw_init", "kvc_wnw_step", "kvc_wnw_chunk_scores",
               "kvc_wnw_update", "kvc_wnw_recall", "kvc_wnw_fixed_select")
KVC_WNW_FIXED = 0
KVC_WNW_ANCHOR = 1
KVC_WNW_TIDAL = 2


KVC_POOL_SEQUENCE = 0
KVC_POOL_LAYER = 1
KVC_SCORE_MEAN = 0
KVC_SCORE_MAX = 1


class kvc_params(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_double), ("rho", ctypes.c_double),
                ("window", ctypes.c_int32), ("base_ratio", ctypes.c_double),
                ("budget_pool", ctypes.c_int32), ("score_pool", ctypes.c_int32)]


class kvc_problem(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("gqa_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_window_q", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("seq_start", ctypes.POINTER(ctypes.c_int64)),
                ("retention", ctypes.POINTER(ctypes.c_double)),
                ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3)]


class kvc_vz_params(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_double), ("n_sink", ctypes.c_int32),
                ("recent_frac", ctypes.c_double)]


class kvc_vz_problem(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("gqa_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity", ctypes.c_int64),
                ("len", ctypes.POINTER(ctypes.c_int64)),
                ("budget", ctypes.POINTER(ctypes.c_int64)),
                ("k_stride", ctypes.c_int64 * 2), ("v_stride", ctypes.c_int64 * 2)]


class kvc_c3_params(ctypes.Structure):
    _fields_ = [("lam", ctypes.c_double), ("r_swaps", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class kvc_c3_problem(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("gqa_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("len", ctypes.POINTER(ctypes.c_int64)),
                ("budget", ctypes.POINTER(ctypes.c_int64)),
                ("k_stride", ctypes.c_int64 * 2), ("v_stride", ctypes.c_int64 * 2),
                ("out_stride", ctypes.c_int64 * 2)]


class kvc_c3_layout(ctypes.Structure):
    _fields_ = [("node_cap", ctypes.c_int64), ("kept_cap", ctypes.c_int64),
                ("index_bytes", ctypes.c_size_t), ("state_bytes", ctypes.c_size_t),
                ("build_workspace_bytes", ctypes.c_size_t),
                ("step_workspace_bytes", ctypes.c_size_t)] + \
        [(f, ctypes.c_size_t) for f in ("start", "size", "left", "parent", "depth", "perm",
                                          "n_nodes", "centroid", "count", "frontier", "ema")]


class kvc_wnw_params(ctypes.Structure):
    _fields_ = [("chunk_len", ctypes.c_int32), ("chunk_stride", ctypes.c_int32),
                ("top_chunks", ctypes.c_int32), ("release_after", ctypes.c_int32)]


class kvc_wnw_problem(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("gqa_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("len", ctypes.POINTER(ctypes.c_int64)),
                ("role", ctypes.POINTER(ctypes.c_uint8)),
                ("k_stride", ctypes.c_int64 * 2), ("host_stride", ctypes.c_int64 * 2),
                ("slot_stride", ctypes.c_int64 * 2)]


class kvc_wnw_layout(ctypes.Structure):
    _fields_ = [("n_anchor", ctypes.c_int32), ("n_tidal", ctypes.c_int32),
                ("block_cap", ctypes.c_int32), ("chunk_cap", ctypes.c_int32),
                ("slot_cap", ctypes.c_int32),
                ("state_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)] + \
        [(f, ctypes.c_size_t) for f in ("idle", "slot_of_block", "block_of_slot", "selected",
                                          "n_recalled", "recalled_block", "recalled_slot")]


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().kvc_status_str(status).decode()
        if status == KVC_ERR_HIP:
            msg += f" (hipError {lib().kvc_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")


_lib = None
_lock = threading.Lock()
_P = ctypes.POINTER
_vp = ctypes.c_void_p


def lib():
    """Load libkvc.so (building it first only if it has never been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not LIB_PATH.exists():
                from audio_kv_cache_amd import build as _b
                _b.build()
            L = ctypes.CDLL(str(LIB_PATH))
            prob, prm = _P(kvc_problem), _P(kvc_params)
            L.kvc_plan.argtypes = [prob, prm, _P(ctypes.c_int64), _P(ctypes.c_size_t)]
            L.kvc_compress.argtypes = [prob, prm, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, ctypes.c_size_t, _vp]
            L.kvc_compress_layers.argtypes = [prob, prm, ctypes.c_int32, ctypes.c_int32, _vp,
                                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              ctypes.c_size_t, _vp]
            L.kvc_scores.argtypes = [prob, prm, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            L.kvc_score_stats.argtypes = [prob, prm, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            L.kvc_score_pool.argtypes = [prob, prm, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            L.kvc_smooth.argtypes = [prob, prm, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            L.kvc_budget.argtypes = [prob, prm, _vp, _vp, _vp, _vp]
            L.kvc_select.argtypes = [prob, prm, _vp, _vp, _vp, _vp, _vp]
            L.kvc_gather.argtypes = [prob, prm, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
            L.kvc_compress_noalloc.argtypes = [prob, prm, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _vp]
            for name in EXPORTS[:11]:
                getattr(L, name).restype = ctypes.c_int
            vp, vq = _P(kvc_vz_problem), _P(kvc_vz_params)
            L.kvc_vz_plan.argtypes = [vp, vq, _P(ctypes.c_int64), _P(ctypes.c_size_t)]
            L.kvc_vz_step.argtypes = [vp, vq, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]
            L.kvc_vz_accumulate.argtypes = [vp, vq, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                            _vp]
            L.kvc_vz_evict.argtypes = [vp, vq, _vp, _vp, _vp]
            L.kvc_vz_gather.argtypes = [vp, vq, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
            L.kvc_vz_step_inplace.argtypes = [vp, vq, _vp, _vp, _vp, _vp, _vp, _vp,
                                              ctypes.c_size_t, _vp]
            for name in VZ_EXPORTS:
                getattr(L, name).restype = ctypes.c_int
            cp, cq = _P(kvc_c3_problem), _P(kvc_c3_params)
            L.kvc_c3_plan.argtypes = [cp, cq, _P(kvc_c3_layout)]
            L.kvc_c3_build.argtypes = [cp, cq, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            L.kvc_c3_step.argtypes = [cp, cq, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]
            L.kvc_c3_score.argtypes = [cp, cq, _vp, _vp, _vp, _vp, _vp]
            L.kvc_c3_select.argtypes = [cp, cq, _vp, _vp, _vp, _vp, _vp]
            L.kvc_c3_update.argtypes = [cp, cq, _vp, _vp, _vp, _vp, _vp]
            L.kvc_c3_gather.argtypes = [cp, cq, _vp, _vp, _vp, _vp, _vp, _vp]
            for name in C3_EXPORTS:
                getattr(L, name).restype = ctypes.c_int
            wp, wq = _P(kvc_wnw_problem), _P(kvc_wnw_params)
            L.kvc_wnw_plan.argtypes = [wp, wq, _P(kvc_wnw_layout)]
            L.kvc_wnw_init.argtypes = [wp, wq, _vp, _vp]
            L.kvc_wnw_step.argtypes = [wp, wq, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_size_t, _vp]
            L.kvc_wnw_chunk_scores.argtypes = [wp, wq, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
            L.kvc_wnw_update.argtypes = [wp, wq, _vp, _vp, _vp, _vp]
            L.kvc_wnw_recall.argtypes = [wp, wq, _vp, _vp, _vp, _vp, _vp, _vp]
            L.kvc_wnw_fixed_select.argtypes = [prob, prm, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                               _vp]
            for name in WNW_EXPORTS:
                getattr(L, name).restype = ctypes.c_int
            L.kvc_status_str.argtypes = [ctypes.c_int]
            L.kvc_status_str.restype = ctypes.c_char_p
            L.kvc_last_hip_error.argtypes = []
            L.kvc_last_hip_error.restype = ctypes.c_int
            _lib = L
    return _lib


def check(status: int, where: str):
    if status != KVC_OK:
        raise KvcError(status, where)
