"""torch-facing wrappers of the C ABI (same names as include/kvc.h).

Only argument marshalling lives here: tensor pointers, strides, the stream,
and output allocation through torch.  The computation is the library's.

Layouts (see include/kvc.h):
  q        [n_seq, n_layers, n_kv_heads * gqa, n_window, head_dim]
  k, v     [n_layers, n_kv_heads, T, head_dim] (any strides with head_dim
           contiguous), sequence i = tokens seq_start[i] .. seq_start[i+1]-1
  S        float32 [n_layers, n_kv_heads]
"""
from __future__ import annotations

import ctypes
import dataclasses

import numpy as np
import torch

from audio_kv_cache_amd import _lib as C


@dataclasses.dataclass
class Params:
    alpha: float = 0.5
    rho: float = 0.7
    window: int = 32
    base_ratio: float = 0.5
    budget_pool: int = C.KVC_POOL_SEQUENCE   # or C.KVC_POOL_LAYER
    score_pool: int = C.KVC_SCORE_MEAN       # or C.KVC_SCORE_MAX

    def c(self) -> C.kvc_params:
        return C.kvc_params(float(self.alpha), float(self.rho), int(self.window),
                            float(self.base_ratio), int(self.budget_pool), int(self.score_pool))


class Spec:
    """Host-side problem description (kvc_problem) and the arrays it points to."""

    def __init__(self, *, n_layers, n_kv_heads, gqa, head_dim, seq_lens, retention,
                 dtype, n_window=32, k_stride=None, v_stride=None):
        self.n_layers, self.n_kv_heads, self.gqa = int(n_layers), int(n_kv_heads), int(gqa)
        self.head_dim, self.n_window = int(head_dim), int(n_window)
        self.dtype = dtype if isinstance(dtype, str) else ("bf16" if dtype == torch.bfloat16 else "f32")
        self.seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
        self.n_seq = int(self.seq_lens.shape[0])
        self._seq_start = np.ascontiguousarray(
            np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int64))
        self._retention = np.ascontiguousarray(np.broadcast_to(
            np.asarray(retention, dtype=np.float64), (self.n_seq,)).copy())
        T = int(self._seq_start[-1])
        dense = (self.n_kv_heads * T * self.head_dim, T * self.head_dim, self.head_dim)
        self.k_stride = tuple(int(x) for x in (k_stride or dense))
        self.v_stride = tuple(int(x) for x in (v_stride or dense))

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def seq_start(self) -> np.ndarray:
        return self._seq_start

    def c(self) -> C.kvc_problem:
        p = C.kvc_problem()
        p.n_seq, p.n_layers, p.n_kv_heads = self.n_seq, self.n_layers, self.n_kv_heads
        p.gqa_group, p.head_dim, p.n_window_q = self.gqa, self.head_dim, self.n_window
        p.dtype = C.KVC_BF16 if self.dtype == "bf16" else C.KVC_F32
        p.seq_start = self._seq_start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        p.retention = self._retention.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        for a in range(3):
            p.k_stride[a] = self.k_stride[a]
            p.v_stride[a] = self.v_stride[a]
        return p

    def score_rows(self) -> int:
        return int(self.n_layers * self.n_kv_heads * self._seq_start[-1])

    def row_offset(self, i: int, l: int, h: int) -> int:
        """First element of unit (i, l, h)'s score row."""
        L = int(self.seq_lens[i])
        return int(self.n_layers * self.n_kv_heads * self._seq_start[i]
                   + (l * self.n_kv_heads + h) * L)

    @staticmethod
    def for_tensors(k, v, *, gqa, seq_lens, retention, n_window=32):
        """Spec for k/v tensors shaped [n_layers, n_kv_heads, T, head_dim]."""
        NL, H, T, d = k.shape
        if k.dtype not in _DTYPES:
            raise ValueError(f"k must be bfloat16 or float32, not {k.dtype}")
        dtype = "bf16" if k.dtype == torch.bfloat16 else "f32"
        return Spec(n_layers=NL, n_kv_heads=H, gqa=gqa, head_dim=d, seq_lens=seq_lens,
                    retention=retention, dtype=dtype, n_window=n_window,
                    k_stride=k.stride()[:3], v_stride=v.stride()[:3])


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# The entry points, one to one.
# ---------------------------------------------------------------------------
def kvc_plan(spec: Spec, params: Params):
    """-> (total_rows, workspace_bytes); host only."""
    rows = ctypes.c_int64(0)
    ws = ctypes.c_size_t(0)
    C.check(C.lib().kvc_plan(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                             ctypes.byref(rows), ctypes.byref(ws)), "kvc_plan")
    return int(rows.value), int(ws.value)


def kvc_compress(spec, params, q, k, v, head_scores, k_out, v_out, idx_out, seg_offsets,
                 budgets, workspace, stream=None):
    C.check(C.lib().kvc_compress(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(head_scores), _ptr(k_out), _ptr(v_out),
                                 _ptr(idx_out), _ptr(seg_offsets), _ptr(budgets),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "kvc_compress")


def kvc_compress_noalloc(spec, params, q, k, v, head_scores, k_out, v_out, idx_out,
                         seg_offsets, budgets, stream=None):
    """kvc_compress with the library's static per-device workspace."""
    C.check(C.lib().kvc_compress_noalloc(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(head_scores),
                                         _ptr(k_out), _ptr(v_out), _ptr(idx_out),
                                         _ptr(seg_offsets), _ptr(budgets), _stream(stream)),
            "kvc_compress_noalloc")


def kvc_compress_layers(spec, params, layer_begin, layer_end, q, k, v, head_scores, k_out,
                        v_out, idx_out, seg_offsets, budgets, workspace, stream=None):
    """q, k, v hold layers [layer_begin, layer_end) only (k, v with spec's
    strides); outputs are the whole problem's."""
    C.check(C.lib().kvc_compress_layers(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                        int(layer_begin), int(layer_end), _ptr(q), _ptr(k),
                                        _ptr(v), _ptr(head_scores), _ptr(k_out), _ptr(v_out),
                                        _ptr(idx_out), _ptr(seg_offsets), _ptr(budgets),
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "kvc_compress_layers")


def kvc_scores(spec, params, q, k, s_out, workspace, stream=None):
    C.check(C.lib().kvc_scores(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(q),
                               _ptr(k), _ptr(s_out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
            "kvc_scores")


def kvc_score_stats(spec, params, q, k, workspace, stream=None):
    C.check(C.lib().kvc_score_stats(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(q),
                                    _ptr(k), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
            "kvc_score_stats")


def kvc_score_pool(spec, params, q, k, s_out, workspace, stream=None):
    C.check(C.lib().kvc_score_pool(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(q),
                                   _ptr(k), _ptr(s_out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
            "kvc_score_pool")


def kvc_smooth(spec, params, s, s_hat, kstar, stream=None, workspace=None):
    """workspace: needed only when a length is not a power of two."""
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    C.check(C.lib().kvc_smooth(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(s),
                               _ptr(s_hat), _ptr(kstar),
                               None if workspace is None else _ptr(workspace), wsb,
                               _stream(stream)), "kvc_smooth")


def kvc_budget(spec, params, head_scores, budgets, seg_offsets, stream=None):
    C.check(C.lib().kvc_budget(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                               _ptr(head_scores), _ptr(budgets), _ptr(seg_offsets),
                               _stream(stream)), "kvc_budget")


def kvc_select(spec, params, s_hat, budgets, seg_offsets, idx_out, stream=None):
    C.check(C.lib().kvc_select(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(s_hat),
                               _ptr(budgets), _ptr(seg_offsets), _ptr(idx_out),
                               _stream(stream)), "kvc_select")


def kvc_gather(spec, params, k, v, idx, seg_offsets, k_out, v_out, stream=None):
    C.check(C.lib().kvc_gather(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(k),
                               _ptr(v), _ptr(idx), _ptr(seg_offsets), _ptr(k_out), _ptr(v_out),
                               _stream(stream)), "kvc_gather")


# ---------------------------------------------------------------------------
# Convenience: allocate outputs with torch and run the whole path.
# ---------------------------------------------------------------------------
def _require_gpu(*ts):
    for t in ts:
        if not (isinstance(t, torch.Tensor) and t.is_cuda):
            raise ValueError("audio_kv_cache_amd needs its tensors in GPU memory")


def allocate(spec: Spec, params: Params, device):
    rows, ws = kvc_plan(spec, params)
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    return dict(
        k_out=torch.empty((rows, spec.head_dim), dtype=tdt, device=device),
        v_out=torch.empty((rows, spec.head_dim), dtype=tdt, device=device),
        idx=torch.empty((rows,), dtype=torch.int32, device=device),
        offsets=torch.empty((spec.n_units + 1,), dtype=torch.int64, device=device),
        budgets=torch.empty((spec.n_units,), dtype=torch.int32, device=device),
        workspace=torch.empty((max(ws, 256),), dtype=torch.uint8, device=device),
    )


_DTYPES = (torch.bfloat16, torch.float32)


def check_compress_args(q, k, v, head_scores, *, gqa, seq_lens) -> None:
    """Reject, before anything reaches the library, tensors whose dtype,
    shape or memory layout the pointers handed to the kernels would not
    match (the C ABI sees only pointers and strides).  Raises ValueError."""
    for name, t in (("q", q), ("k", k), ("v", v), ("head_scores", head_scores)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
    if k.dtype not in _DTYPES:
        raise ValueError(f"k must be bfloat16 or float32, not {k.dtype}")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError(f"q, k and v must share one dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    if k.dim() != 4 or v.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must both be [n_layers, n_kv_heads, T, head_dim]")
    if k.stride(-1) != 1 or v.stride(-1) != 1:
        raise ValueError("k and v need head_dim contiguous (stride(-1) == 1)")
    NL, H, T, d = (int(x) for x in k.shape)
    lens = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    if lens.size == 0 or (lens < 0).any() or int(lens.sum()) > T:
        raise ValueError(f"seq_lens must be >= 0 with sum(seq_lens) <= T = {T}")
    if q.dim() < 2 or int(q.shape[-1]) != d:
        raise ValueError("q's last dimension must be head_dim")
    nwin = int(q.shape[-2])
    want = lens.size * NL * H * int(gqa) * nwin * d
    if not q.is_contiguous() or q.numel() != want:
        raise ValueError(f"q must be contiguous with n_seq*n_layers*n_kv_heads*gqa*n_window*"
                         f"head_dim = {want} elements")
    if head_scores.dtype != torch.float32 or not head_scores.is_contiguous() \
            or head_scores.numel() != NL * H:
        raise ValueError(f"head_scores must be contiguous float32 [{NL}, {H}]")
    devs = {t.device for t in (q, k, v, head_scores)}
    if len(devs) != 1:
        raise ValueError("q, k, v and head_scores must be on one device")


def compress(q, k, v, head_scores, *, gqa, seq_lens, retention, alpha=0.5, rho=0.7,
             window=32, base_ratio=0.5, budget_pool=C.KVC_POOL_SEQUENCE,
             score_pool=C.KVC_SCORE_MEAN, out=None, stream=None):
    """Whole path; returns dict(k_out, v_out, idx, offsets, budgets, workspace)."""
    check_compress_args(q, k, v, head_scores, gqa=gqa, seq_lens=seq_lens)
    _require_gpu(q, k, v, head_scores)
    spec = Spec.for_tensors(k, v, gqa=gqa, seq_lens=seq_lens, retention=retention,
                            n_window=q.shape[-2])
    params = Params(alpha, rho, window, base_ratio, budget_pool, score_pool)
    if out is None:
        o = allocate(spec, params, k.device)
    else:
        o = out
        rows, ws = kvc_plan(spec, params)
        need = dict(k_out=(k.dtype, rows * spec.head_dim), v_out=(k.dtype, rows * spec.head_dim),
                    idx=(torch.int32, rows), offsets=(torch.int64, spec.n_units + 1),
                    budgets=(torch.int32, spec.n_units), workspace=(torch.uint8, ws))
        for name, (dt, n) in need.items():
            t = o.get(name)
            if not isinstance(t, torch.Tensor) or t.dtype != dt or not t.is_contiguous() \
                    or t.numel() < n or t.device != k.device:
                raise ValueError(f"out[{name!r}] must be a contiguous {dt} tensor of at least "
                                 f"{n} elements on {k.device}")
    kvc_compress(spec, params, q, k, v, head_scores, o["k_out"], o["v_out"], o["idx"],
                 o["offsets"], o["budgets"], o["workspace"], stream)
    return o


# ---------------------------------------------------------------------------
# Decode-time decayed eviction (include/kvc_voxzip.h)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class VzParams:
    gamma: float = 0.95
    n_sink: int = 4
    recent_frac: float = 0.2

    def c(self) -> C.kvc_vz_params:
        return C.kvc_vz_params(float(self.gamma), int(self.n_sink), float(self.recent_frac))


class VzSpec:
    """Host-side kvc_vz_problem: caches [units][capacity][head_dim] for K and V
    (or any strides with head_dim contiguous), per-sequence lengths and
    budgets."""

    def __init__(self, *, n_layers, n_kv_heads, gqa, head_dim, lens, budgets, capacity,
                 dtype, k_stride=None, v_stride=None):
        self.n_layers, self.n_kv_heads, self.gqa = int(n_layers), int(n_kv_heads), int(gqa)
        self.head_dim, self.capacity = int(head_dim), int(capacity)
        self.dtype = dtype if isinstance(dtype, str) else ("bf16" if dtype == torch.bfloat16 else "f32")
        self._len = np.ascontiguousarray(np.asarray(lens, dtype=np.int64).reshape(-1))
        self.n_seq = int(self._len.shape[0])
        self._budget = np.ascontiguousarray(np.broadcast_to(
            np.asarray(budgets, dtype=np.int64), (self.n_seq,)).copy())
        dense = (self.capacity * self.head_dim, self.head_dim)
        self.k_stride = tuple(int(x) for x in (k_stride or dense))
        self.v_stride = tuple(int(x) for x in (v_stride or dense))

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def lens(self) -> np.ndarray:
        return self._len

    @property
    def budgets(self) -> np.ndarray:
        return self._budget

    def c(self) -> C.kvc_vz_problem:
        p = C.kvc_vz_problem()
        p.n_seq, p.n_layers, p.n_kv_heads = self.n_seq, self.n_layers, self.n_kv_heads
        p.gqa_group, p.head_dim = self.gqa, self.head_dim
        p.dtype = C.KVC_BF16 if self.dtype == "bf16" else C.KVC_F32
        p.capacity = self.capacity
        p.len = self._len.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        p.budget = self._budget.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        for a in range(2):
            p.k_stride[a] = self.k_stride[a]
            p.v_stride[a] = self.v_stride[a]
        return p


def kvc_vz_plan(spec: VzSpec, params: VzParams):
    """-> (new_len [n_seq] int64, workspace_bytes); host only."""
    nl = np.zeros(spec.n_seq, dtype=np.int64)
    ws = ctypes.c_size_t(0)
    C.check(C.lib().kvc_vz_plan(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                nl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                ctypes.byref(ws)), "kvc_vz_plan")
    return nl, int(ws.value)


def kvc_vz_step(spec, params, q, k, v, a_prev, k_out, v_out, a_out, idx_out, workspace,
                stream=None):
    C.check(C.lib().kvc_vz_step(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(q),
                                _ptr(k), _ptr(v), _ptr(a_prev), _ptr(k_out), _ptr(v_out),
                                _ptr(a_out), _ptr(idx_out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
            "kvc_vz_step")


def kvc_vz_step_inplace(spec, params, q, k, a, pos, free_slot, workspace, stream=None):
    """Decode step with the cache kept in its slots (a, pos updated in place)."""
    C.check(C.lib().kvc_vz_step_inplace(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                        _ptr(q), _ptr(k), _ptr(a), _ptr(pos), _ptr(free_slot),
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "kvc_vz_step_inplace")


def kvc_vz_accumulate(spec, params, q, k, a_prev, a, workspace, stream=None):
    C.check(C.lib().kvc_vz_accumulate(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                      _ptr(q), _ptr(k), _ptr(a_prev), _ptr(a), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "kvc_vz_accumulate")


def kvc_vz_evict(spec, params, a, idx_out, stream=None):
    C.check(C.lib().kvc_vz_evict(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(a),
                                 _ptr(idx_out), _stream(stream)), "kvc_vz_evict")


def kvc_vz_gather(spec, params, k, v, a, idx, k_out, v_out, a_out, stream=None):
    C.check(C.lib().kvc_vz_gather(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(k),
                                  _ptr(v), _ptr(a), _ptr(idx), _ptr(k_out), _ptr(v_out),
                                  _ptr(a_out), _stream(stream)), "kvc_vz_gather")


# ---------------------------------------------------------------------------
# Query-guided retrieval (include/kvc_c3.h)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class C3Params:
    lam: float = 0.5
    r_swaps: int = 2
    seed: int = 0

    def c(self) -> C.kvc_c3_params:
        return C.kvc_c3_params(float(self.lam), int(self.r_swaps), int(self.seed))


class C3Spec:
    """Host-side kvc_c3_problem: bf16 key/value caches [units][capacity][head_dim]
    (or any strides with head_dim contiguous), per-sequence audio lengths n and
    budgets B, output rows [units][out_rows][head_dim]."""

    def __init__(self, *, n_layers, n_kv_heads, gqa, head_dim, lens, budgets, capacity,
                 k_stride=None, v_stride=None, out_stride=None):
        self.n_layers, self.n_kv_heads, self.gqa = int(n_layers), int(n_kv_heads), int(gqa)
        self.head_dim, self.capacity = int(head_dim), int(capacity)
        self._len = np.ascontiguousarray(np.asarray(lens, dtype=np.int64).reshape(-1))
        self.n_seq = int(self._len.shape[0])
        self._budget = np.ascontiguousarray(np.broadcast_to(
            np.asarray(budgets, dtype=np.int64), (self.n_seq,)).copy())
        dense = (self.capacity * self.head_dim, self.head_dim)
        self.k_stride = tuple(int(x) for x in (k_stride or dense))
        self.v_stride = tuple(int(x) for x in (v_stride or dense))
        self.out_rows = int(max(1, np.minimum(self._len, self._budget).max()))
        self.out_stride = tuple(int(x) for x in (out_stride or
                                                  (self.out_rows * self.head_dim, self.head_dim)))

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def lens(self) -> np.ndarray:
        return self._len

    @property
    def budgets(self) -> np.ndarray:
        return self._budget

    def c(self) -> C.kvc_c3_problem:
        p = C.kvc_c3_problem()
        p.n_seq, p.n_layers, p.n_kv_heads = self.n_seq, self.n_layers, self.n_kv_heads
        p.gqa_group, p.head_dim, p.capacity = self.gqa, self.head_dim, self.capacity
        p.len = self._len.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        p.budget = self._budget.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        for a in range(2):
            p.k_stride[a] = self.k_stride[a]
            p.v_stride[a] = self.v_stride[a]
            p.out_stride[a] = self.out_stride[a]
        return p


def kvc_c3_plan(spec: C3Spec, params: C3Params) -> C.kvc_c3_layout:
    lay = C.kvc_c3_layout()
    C.check(C.lib().kvc_c3_plan(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                ctypes.byref(lay)), "kvc_c3_plan")
    return lay


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def kvc_c3_build(spec, params, k, index, state, workspace, stream=None):
    C.check(C.lib().kvc_c3_build(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(k),
                                 _ptr(index), _ptr(state), _ptr(workspace), _nbytes(workspace),
                                 _stream(stream)), "kvc_c3_build")


def kvc_c3_step(spec, params, index, state_in, state_out, q, k, v, k_out, v_out, idx_out,
                workspace, stream=None):
    C.check(C.lib().kvc_c3_step(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(index),
                                _ptr(state_in), _ptr(state_out), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(k_out), _ptr(v_out), _ptr(idx_out), _ptr(workspace),
                                _nbytes(workspace), _stream(stream)), "kvc_c3_step")


def kvc_c3_score(spec, params, index, state, q, sigma, stream=None):
    C.check(C.lib().kvc_c3_score(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(index),
                                 _ptr(state), _ptr(q), _ptr(sigma), _stream(stream)),
            "kvc_c3_score")


def kvc_c3_select(spec, params, index, state, sigma, idx_out, stream=None):
    C.check(C.lib().kvc_c3_select(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                  _ptr(index), _ptr(state), _ptr(sigma), _ptr(idx_out),
                                  _stream(stream)), "kvc_c3_select")


def kvc_c3_update(spec, params, index, state_in, sigma, state_out, stream=None):
    C.check(C.lib().kvc_c3_update(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                  _ptr(index), _ptr(state_in), _ptr(sigma), _ptr(state_out),
                                  _stream(stream)), "kvc_c3_update")


def kvc_c3_gather(spec, params, k, v, idx, k_out, v_out, stream=None):
    C.check(C.lib().kvc_c3_gather(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(k),
                                  _ptr(v), _ptr(idx), _ptr(k_out), _ptr(v_out),
                                  _stream(stream)), "kvc_c3_gather")


class C3Views:
    """torch views of an index and a state buffer (uint8 device tensors) by
    the layout's offsets."""

    def __init__(self, spec: C3Spec, lay, index, state):
        U, NC, CAP, D = spec.n_units, int(lay.node_cap), spec.capacity, spec.head_dim

        def view(buf, off, count, dtype, shape):
            esz = torch.empty((), dtype=dtype).element_size()
            return buf[off:off + count * esz].view(dtype).view(*shape)
        self.start = view(index, lay.start, U * NC, torch.int32, (U, NC))
        self.size = view(index, lay.size, U * NC, torch.int32, (U, NC))
        self.left = view(index, lay.left, U * NC, torch.int32, (U, NC))
        self.parent = view(index, lay.parent, U * NC, torch.int32, (U, NC))
        self.depth = view(index, lay.depth, U * NC, torch.int32, (U, NC))
        self.perm = view(index, lay.perm, U * CAP, torch.int32, (U, CAP))
        self.n_nodes = view(index, lay.n_nodes, U, torch.int32, (U,))
        self.centroid = view(index, lay.centroid, U * NC * D, torch.int16, (U, NC, D))
        self.count = view(state, lay.count, U, torch.int32, (U,))
        self.frontier = view(state, lay.frontier, U * CAP, torch.int32, (U, CAP))
        self.ema = view(state, lay.ema, U * CAP, torch.float64, (U, CAP))


def c3_allocate(spec: C3Spec, params: C3Params, device):
    """Index, two states, workspaces and outputs for a C3 problem."""
    lay = kvc_c3_plan(spec, params)
    U, R, D = spec.n_units, spec.out_rows, spec.head_dim

    def buf(n):
        return torch.empty((max(int(n), 256),), dtype=torch.uint8, device=device)
    return dict(
        layout=lay,
        index=buf(lay.index_bytes),
        state=[buf(lay.state_bytes), buf(lay.state_bytes)],
        build_ws=buf(lay.build_workspace_bytes),
        step_ws=buf(lay.step_workspace_bytes),
        k_out=torch.empty((U, R, D), dtype=torch.bfloat16, device=device),
        v_out=torch.empty((U, R, D), dtype=torch.bfloat16, device=device),
        idx=torch.empty((U, int(lay.kept_cap)), dtype=torch.int32, device=device),
        sigma=torch.empty((U, spec.capacity), dtype=torch.float32, device=device),
    )


# ---------------------------------------------------------------------------
# WnW chunk recall (include/kvc_wnw.h)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class WnwParams:
    chunk_len: int = 50       # 4 s at 12.5 audio tokens per second
    chunk_stride: int = 25    # 2 s
    top_chunks: int = 3
    release_after: int = 3

    def c(self) -> C.kvc_wnw_params:
        return C.kvc_wnw_params(int(self.chunk_len), int(self.chunk_stride),
                                int(self.top_chunks), int(self.release_after))

    @property
    def slot_cap(self) -> int:
        return self.top_chunks * self.release_after * (self.chunk_len // self.chunk_stride)


class WnwSpec:
    """Host-side kvc_wnw_problem: per-sequence audio lengths, a role per KV
    head (0 fixed, 1 anchor, 2 tidal), the anchors' device keys, the tidal
    heads' page-locked host copies and device slot buffers (dense
    [units][rows][head_dim] strides by default)."""

    def __init__(self, *, n_layers, n_kv_heads, gqa, head_dim, lens, roles, capacity,
                 slot_rows, k_stride=None, host_stride=None, slot_stride=None):
        self.n_layers, self.n_kv_heads, self.gqa = int(n_layers), int(n_kv_heads), int(gqa)
        self.head_dim, self.capacity = int(head_dim), int(capacity)
        self._len = np.ascontiguousarray(np.asarray(lens, dtype=np.int64).reshape(-1))
        self.n_seq = int(self._len.shape[0])
        self._role = np.ascontiguousarray(np.asarray(roles, dtype=np.uint8).reshape(-1))
        assert self._role.shape[0] == self.n_layers * self.n_kv_heads
        dense = (self.capacity * self.head_dim, self.head_dim)
        self.k_stride = tuple(int(x) for x in (k_stride or dense))
        self.host_stride = tuple(int(x) for x in (host_stride or dense))
        self.slot_rows = int(slot_rows)
        self.slot_stride = tuple(int(x) for x in (slot_stride or
                                                   (self.slot_rows * self.head_dim, self.head_dim)))

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def lens(self) -> np.ndarray:
        return self._len

    @property
    def roles(self) -> np.ndarray:
        return self._role

    def c(self) -> C.kvc_wnw_problem:
        p = C.kvc_wnw_problem()
        p.n_seq, p.n_layers, p.n_kv_heads = self.n_seq, self.n_layers, self.n_kv_heads
        p.gqa_group, p.head_dim, p.capacity = self.gqa, self.head_dim, self.capacity
        p.len = self._len.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        p.role = self._role.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        for a in range(2):
            p.k_stride[a] = self.k_stride[a]
            p.host_stride[a] = self.host_stride[a]
            p.slot_stride[a] = self.slot_stride[a]
        return p


def kvc_wnw_plan(spec: WnwSpec, params: WnwParams) -> C.kvc_wnw_layout:
    lay = C.kvc_wnw_layout()
    C.check(C.lib().kvc_wnw_plan(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                 ctypes.byref(lay)), "kvc_wnw_plan")
    return lay


def kvc_wnw_init(spec, params, state, stream=None):
    C.check(C.lib().kvc_wnw_init(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(state),
                                 _stream(stream)), "kvc_wnw_init")


def _hptr(t):
    return None if t is None else t.data_ptr()


def kvc_wnw_step(spec, params, q, k, state_in, state_out, host_k, host_v, slot_k, slot_v,
                 sigma, workspace, stream=None):
    C.check(C.lib().kvc_wnw_step(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(q),
                                 _ptr(k), _ptr(state_in), _ptr(state_out), _hptr(host_k),
                                 _hptr(host_v), _hptr(slot_k), _hptr(slot_v), _hptr(sigma),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)),
            "kvc_wnw_step")


def kvc_wnw_chunk_scores(spec, params, q, k, sigma, workspace, stream=None):
    C.check(C.lib().kvc_wnw_chunk_scores(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                         _ptr(q), _ptr(k), _ptr(sigma), _ptr(workspace),
                                         _nbytes(workspace), _stream(stream)),
            "kvc_wnw_chunk_scores")


def kvc_wnw_update(spec, params, sigma, state_in, state_out, stream=None):
    C.check(C.lib().kvc_wnw_update(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(sigma),
                                   _ptr(state_in), _ptr(state_out), _stream(stream)),
            "kvc_wnw_update")


def kvc_wnw_recall(spec, params, state, host_k, host_v, slot_k, slot_v, stream=None):
    C.check(C.lib().kvc_wnw_recall(ctypes.byref(spec.c()), ctypes.byref(params.c()), _ptr(state),
                                   _hptr(host_k), _hptr(host_v), _hptr(slot_k), _hptr(slot_v),
                                   _stream(stream)), "kvc_wnw_recall")


def kvc_wnw_fixed_select(spec: Spec, params: Params, seg_len, s_hat, budgets, seg_offsets,
                         idx_out, stream=None):
    C.check(C.lib().kvc_wnw_fixed_select(ctypes.byref(spec.c()), ctypes.byref(params.c()),
                                         int(seg_len), _ptr(s_hat), _ptr(budgets),
                                         _ptr(seg_offsets), _ptr(idx_out), _stream(stream)),
            "kvc_wnw_fixed_select")


class WnwViews:
    """torch views of a WnW state buffer (uint8 device tensor) by the
    layout's offsets."""

    def __init__(self, spec: WnwSpec, params: WnwParams, lay, state):
        N = spec.n_seq

        def view(off, cols):
            return state[off:off + 4 * N * cols].view(torch.int32).view(N, cols)
        self.idle = view(lay.idle, int(lay.chunk_cap))
        self.slot_of_block = view(lay.slot_of_block, int(lay.block_cap))
        self.block_of_slot = view(lay.block_of_slot, int(lay.slot_cap))
        self.selected = view(lay.selected, int(params.top_chunks))
        self.n_recalled = view(lay.n_recalled, 1).view(N)
        self.recalled_block = view(lay.recalled_block, int(lay.slot_cap))
        self.recalled_slot = view(lay.recalled_slot, int(lay.slot_cap))


def wnw_allocate(spec: WnwSpec, params: WnwParams, device):
    """Two states, a workspace, chunk scores and slot buffers for a WnW problem."""
    lay = kvc_wnw_plan(spec, params)

    def buf(n):
        return torch.empty((max(int(n), 256),), dtype=torch.uint8, device=device)
    U, D = spec.n_units, spec.head_dim
    return dict(
        layout=lay,
        state=[buf(lay.state_bytes), buf(lay.state_bytes)],
        ws=buf(lay.workspace_bytes),
        sigma=torch.zeros((spec.n_seq, int(lay.chunk_cap)), dtype=torch.float32, device=device),
        slot_k=torch.zeros((U, spec.slot_rows, D), dtype=torch.bfloat16, device=device),
        slot_v=torch.zeros((U, spec.slot_rows, D), dtype=torch.bfloat16, device=device),
    )
