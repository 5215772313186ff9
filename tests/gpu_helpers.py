"""Shared plumbing for the GPU parity tests: synthetic problems to device
tensors, one call per C-ABI entry point, and the parity criteria.

Criteria (tolerances are the ones the scoring/smoothing arithmetic allows:
bf16 inputs with fp32 accumulation 1e-3, fp32 inputs 1e-5, norm-wise):
  * rows s and s_hat: max|x - ref| / max|ref| <= TOL
  * k*: equal, unless the oracle's energy at the smaller of the two cutoffs is
    within TAU * E(n) of rho * E(n) (the cutoff is a threshold decision on a
    prefix sum: a rounding-sized change may move it); s_hat is then compared
    with the oracle re-run at the GPU's k*
  * budgets, offsets, indices on identical scores, gathered rows: bit-exact
  * end to end: a kept/dropped disagreement is allowed only at positions
    whose oracle s_hat lies within TOL * max|s_hat| of the unit's threshold.
"""
from __future__ import annotations

import numpy as np
import torch

from audio_kv_cache_amd import api, synth
from oracle import oracle as O

TOL = {"bf16": 1e-3, "f32": 1e-5}
TAU = {"bf16": 2e-3, "f32": 2e-5}


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class Dev:
    """A synthetic problem resident in GPU memory."""

    def __init__(self, prob: synth.Problem):
        self.prob = prob
        cfg, hdr = prob.cfg, prob.hdr
        self.cfg, self.hdr = cfg, hdr
        self.dtype = cfg.dtype
        self.q = to_torch(prob.q, cfg.dtype)
        self.k = to_torch(prob.k, cfg.dtype)
        self.v = to_torch(prob.v, cfg.dtype)
        self.S = torch.from_numpy(np.ascontiguousarray(hdr.head_scores)).cuda()
        self.spec = api.Spec.for_tensors(self.k, self.v, gqa=cfg.gqa, seq_lens=hdr.lengths,
                                         retention=hdr.retention, n_window=cfg.n_window)
        self.params = api.Params(cfg.alpha, cfg.rho, cfg.window, cfg.base_ratio,
                                 cfg.budget_pool, cfg.score_pool)
        self.rows, self.ws_bytes = api.kvc_plan(self.spec, self.params)

    def units(self):
        c = self.cfg
        return [(i, l, h) for i in range(c.n_seq) for l in range(c.n_layers)
                for h in range(c.n_kv_heads)]

    def uindex(self, i, l, h):
        return O.unit_index(self.cfg, i, l, h)

    def row(self, flat: np.ndarray, i, l, h):
        o = self.spec.row_offset(i, l, h)
        return flat[o:o + int(self.hdr.lengths[i])]

    # -- entry points ------------------------------------------------------
    def budget(self):
        b = torch.empty(self.spec.n_units, dtype=torch.int32, device="cuda")
        off = torch.empty(self.spec.n_units + 1, dtype=torch.int64, device="cuda")
        api.kvc_budget(self.spec, self.params, self.S, b, off)
        torch.cuda.synchronize()
        return b.cpu().numpy(), off.cpu().numpy()

    def scores(self):
        s = torch.empty(self.spec.score_rows(), dtype=torch.float32, device="cuda")
        ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        api.kvc_scores(self.spec, self.params, self.q, self.k, s, ws)
        torch.cuda.synchronize()
        return s.cpu().numpy()

    def scores_two_pass(self):
        """Step 1 through kvc_score_stats then kvc_score_pool."""
        s = torch.empty(self.spec.score_rows(), dtype=torch.float32, device="cuda")
        ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        api.kvc_score_stats(self.spec, self.params, self.q, self.k, ws)
        api.kvc_score_pool(self.spec, self.params, self.q, self.k, s, ws)
        torch.cuda.synchronize()
        return s.cpu().numpy()

    def smooth(self, s_flat: np.ndarray):
        s = torch.from_numpy(np.ascontiguousarray(s_flat, dtype=np.float32)).cuda()
        sh = torch.empty_like(s)
        ks = torch.empty(self.spec.n_units, dtype=torch.int32, device="cuda")
        ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device="cuda")
        api.kvc_smooth(self.spec, self.params, s, sh, ks, workspace=ws)
        torch.cuda.synchronize()
        return sh.cpu().numpy(), ks.cpu().numpy()

    def select(self, sh_flat: np.ndarray, budgets: np.ndarray, offsets: np.ndarray):
        sh = torch.from_numpy(np.ascontiguousarray(sh_flat, dtype=np.float32)).cuda()
        b = torch.from_numpy(np.ascontiguousarray(budgets, dtype=np.int32)).cuda()
        off = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int64)).cuda()
        idx = torch.full((int(offsets[-1]),), -1, dtype=torch.int32, device="cuda")
        api.kvc_select(self.spec, self.params, sh, b, off, idx)
        torch.cuda.synchronize()
        return idx.cpu().numpy()

    def gather(self, idx: np.ndarray, offsets: np.ndarray):
        i = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
        off = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int64)).cuda()
        tdt = self.k.dtype
        ko = torch.empty((self.rows, self.cfg.head_dim), dtype=tdt, device="cuda")
        vo = torch.empty_like(ko)
        api.kvc_gather(self.spec, self.params, self.k, self.v, i, off, ko, vo)
        torch.cuda.synchronize()
        return to_numpy(ko, self.dtype), to_numpy(vo, self.dtype)

    def compress(self, out=None):
        o = api.compress(self.q, self.k, self.v, self.S, gqa=self.cfg.gqa,
                         seq_lens=self.hdr.lengths, retention=self.hdr.retention,
                         alpha=self.cfg.alpha, rho=self.cfg.rho, window=self.cfg.window,
                         base_ratio=self.cfg.base_ratio, budget_pool=self.cfg.budget_pool,
                         score_pool=self.cfg.score_pool, out=out)
        torch.cuda.synchronize()
        return o


def check_kstar(ks_gpu: int, ks_ref: int, energy_ref: np.ndarray, rho: float, dtype: str):
    """True when the cutoffs agree or differ only inside the ambiguity band."""
    if ks_gpu == ks_ref:
        return True
    k = min(ks_gpu, ks_ref)
    En = energy_ref[-1]
    return abs(energy_ref[k] - rho * En) <= TAU[dtype] * En


def check_smoothed_row(s_row32: np.ndarray, sh_gpu: np.ndarray, ks_gpu: int, alpha, rho,
                       dtype: str):
    """Compare one GPU s_hat row with the oracle on the same fp32 input row."""
    sh_ref, ks_ref, E, _ = O.sss(s_row32.astype(np.float64), alpha, rho)
    assert check_kstar(ks_gpu, ks_ref, E, rho, dtype), (ks_gpu, ks_ref)
    if ks_gpu != ks_ref:
        sh_ref = O.sss(s_row32.astype(np.float64), alpha, rho, kstar=ks_gpu)[0]
    err = rel_err(sh_gpu, sh_ref)
    assert err <= TOL[dtype], err
    return err, ks_ref


def check_kept_sets(idx_gpu: np.ndarray, kept_ref: np.ndarray, sh_ref: np.ndarray, b: int,
                    window: int, dtype: str):
    """End-to-end criterion for one unit."""
    L = sh_ref.shape[0]
    assert idx_gpu.shape[0] == b == kept_ref.shape[0]
    assert np.all(np.diff(idx_gpu) > 0)
    assert idx_gpu[-window:].tolist() == list(range(L - window, L)) if window else True
    k = b - window
    if k <= 0 or k >= L - window:
        assert np.array_equal(idx_gpu, kept_ref)
        return 0
    cand = sh_ref[:L - window]
    theta = np.sort(cand)[::-1][k - 1]
    diff = np.setxor1d(idx_gpu, kept_ref)
    tol = TOL[dtype] * np.max(np.abs(sh_ref))
    bad = [j for j in diff if abs(sh_ref[j] - theta) > tol]
    assert not bad, (len(diff), bad[:10])
    return len(diff)
