"""GPU parity of WnW chunk recall (include/kvc_wnw.h) against oracle/wnw.py.

Criteria: chunk scores within 1e-4 of the largest (fp32 sums of fp32
probabilities against fp64); every decision bit-exact given the GPU's own
scores (the oracle's top-K and residency update run on them: selected
chunks, idle counts, slot maps, recall lists); slot contents bit-exact
against the host copies; fixed-head segment selection bit-exact.
"""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from audio_kv_cache_amd import _lib as C  # noqa: E402
from audio_kv_cache_amd import api, synth  # noqa: E402
from oracle import wnw as W  # noqa: E402

pytestmark = pytest.mark.gpu

SIGMA_TOL = 1e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _pinned(bits: np.ndarray):
    t = torch.empty(bits.shape, dtype=torch.int16, pin_memory=True)
    t.copy_(torch.from_numpy(bits.view(np.int16)))
    return t


class WnwDev:
    def __init__(self, cfg: synth.WnwConfig, params: api.WnwParams, fast_host=False):
        self.cfg, self.params = cfg, params
        self.roles = synth.wnw_roles(cfg)
        S = params.chunk_stride
        self.spec = api.WnwSpec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                                head_dim=cfg.head_dim, lens=cfg.lens, roles=self.roles,
                                capacity=cfg.capacity, slot_rows=params.slot_cap * S)
        self.kh, self.vh = synth.wnw_host_copies(cfg, fast=fast_host)
        self.ka = synth.wnw_anchor_keys(cfg)
        if fast_host:
            # random bits for the tidal copies; the anchors' device rows from
            # the cache model
            kd = np.zeros_like(self.kh)
            upseq = cfg.n_layers * cfg.n_kv_heads
            for i in range(cfg.n_seq):
                for a, un in enumerate(sorted(cfg.anchors)):
                    kd[i * upseq + un] = self.ka[i, a]
        else:
            kd = self.kh
        self.k = torch.from_numpy(kd.view(np.int16)).cuda()
        self.hk, self.hv = _pinned(self.kh), _pinned(self.vh)
        self.buf = api.wnw_allocate(self.spec, params, "cuda")
        self.lay = self.buf["layout"]
        for st in self.buf["state"]:      # (both: padding between regions compares equal)
            api.kvc_wnw_init(self.spec, params, st)
        torch.cuda.synchronize()
        self.cur = 0
        self.ref = [W.Residency(int(n), S, params.chunk_len, params.top_chunks,
                                params.release_after) for n in cfg.lens]
        self.n_recalls = self.n_releases = 0

    def queries(self, step):
        return synth.wnw_queries(self.cfg, step, self.ka)

    def views(self, which):
        return api.WnwViews(self.spec, self.params, self.lay, self.buf["state"][which])

    def step(self, step, staged=False):
        q = torch.from_numpy(self.queries(step).view(np.int16)).cuda()
        si, so = self.buf["state"][self.cur], self.buf["state"][1 - self.cur]
        b = self.buf
        if staged:
            api.kvc_wnw_chunk_scores(self.spec, self.params, q, self.k, b["sigma"], b["ws"])
            api.kvc_wnw_update(self.spec, self.params, b["sigma"], si, so)
            api.kvc_wnw_recall(self.spec, self.params, so, self.hk, self.hv, b["slot_k"],
                               b["slot_v"])
        else:
            api.kvc_wnw_step(self.spec, self.params, q, self.k, si, so, self.hk, self.hv,
                             b["slot_k"], b["slot_v"], b["sigma"], b["ws"])
        torch.cuda.synchronize()
        self.cur = 1 - self.cur
        return q

    def check_step(self, step, staged=False):
        cfg, prm = self.cfg, self.params
        S, Wc = prm.chunk_stride, prm.chunk_len
        self.step(step, staged)
        sig = self.buf["sigma"].cpu().numpy()
        v = self.views(self.cur)
        idle = v.idle.cpu().numpy()
        sob = v.slot_of_block.cpu().numpy()
        bos = v.block_of_slot.cpu().numpy()
        sel = v.selected.cpu().numpy()
        nrec = v.n_recalled.cpu().numpy()
        rb = v.recalled_block.cpu().numpy()
        rs = v.recalled_slot.cpu().numpy()
        qa = synth.bf16_bits_to_f32(self.queries(step))
        for i, n in enumerate(cfg.lens):
            n = int(n)
            C_i = W.n_chunks(n, S, Wc)
            ks = [synth.bf16_bits_to_f32(self.ka[i, a, :n]) for a in range(len(cfg.anchors))]
            want = W.chunk_scores(list(qa[i]), ks, n, S, Wc)
            got = sig[i, :C_i].astype(np.float64)
            err = np.max(np.abs(got - want)) / np.max(want)
            assert err <= SIGMA_TOL, (i, err)
            # decisions from the GPU's scores
            sel_ref = W.top_chunks(got, prm.top_chunks)
            assert sel[i, :len(sel_ref)].tolist() == sel_ref, (i, step)
            assert np.all(sel[i, len(sel_ref):] == -1)
            prev = self.ref[i]
            self.ref[i], rec = W.update(prev, sel_ref)
            r = self.ref[i]
            self.n_recalls += len(rec)
            self.n_releases += sum(1 for a, b in zip(prev.slot_of_block, r.slot_of_block)
                                   if a >= 0 and b < 0)
            assert idle[i, :C_i].tolist() == r.idle and np.all(idle[i, C_i:] == -1)
            B_i = W.n_blocks(n, S)
            assert sob[i, :B_i].tolist() == r.slot_of_block and np.all(sob[i, B_i:] == -1)
            cap = r.slot_cap()
            assert bos[i, :cap].tolist() == r.block_of_slot and np.all(bos[i, cap:] == -1)
            assert int(nrec[i]) == len(rec)
            assert list(zip(rb[i, :len(rec)].tolist(), rs[i, :len(rec)].tolist())) == rec
        return self.check_slots()

    def check_slots(self):
        cfg, S = self.cfg, self.params.chunk_stride
        sk = self.buf["slot_k"].view(torch.int16).cpu().numpy().view(np.uint16)
        sv = self.buf["slot_v"].view(torch.int16).cpu().numpy().view(np.uint16)
        upseq = cfg.n_layers * cfg.n_kv_heads
        for i, n in enumerate(cfg.lens):
            r = self.ref[i]
            for u0 in range(upseq):
                u = i * upseq + u0
                if self.roles[u0] != 2:
                    assert not sk[u].any() and not sv[u].any()   # never written
                    continue
                for b, s in enumerate(r.slot_of_block):
                    if s >= 0:
                        lo, hi = W.block_range(b, int(n), S)
                        rows = slice(s * S, s * S + hi - lo)
                        assert np.array_equal(sk[u, rows], self.kh[u, lo:hi]), (u, b, s)
                        assert np.array_equal(sv[u, rows], self.vh[u, lo:hi]), (u, b, s)
        return True


@pytest.mark.parametrize("name", ["wnw_tiny", "wnw_mixed", "wnw_edge", "wnw_g20", "wnw_g32"])
def test_steps_match_oracle(name):
    say(f"[wnw] {name}")
    D = WnwDev(synth.WNW_CONFIGS[name], api.WnwParams())
    for t in range(40):
        D.check_step(t)
    say(f"    {D.n_recalls} blocks recalled, {D.n_releases} released")
    assert D.n_recalls > 0
    if name != "wnw_edge":   # (there every block fits the slots and stays)
        assert D.n_releases > 0


@pytest.mark.parametrize("prm", [dict(top_chunks=1, release_after=1),
                                 dict(top_chunks=8, release_after=8, chunk_len=25),
                                 dict(chunk_len=75, top_chunks=2, release_after=2),
                                 dict(chunk_len=20, chunk_stride=10, top_chunks=3)])
def test_parameter_variants(prm):
    say(f"[wnw] mixed {prm}")
    D = WnwDev(synth.WNW_CONFIGS["wnw_mixed"], api.WnwParams(**prm))
    for t in range(24):
        D.check_step(t)


def test_stage_entry_points_equal_the_step():
    cfg = synth.WNW_CONFIGS["wnw_mixed"]
    A = WnwDev(cfg, api.WnwParams())
    B = WnwDev(cfg, api.WnwParams())
    for t in range(10):
        A.step(t)
        B.step(t, staged=True)
        assert torch.equal(A.buf["sigma"], B.buf["sigma"])
        assert torch.equal(A.buf["state"][A.cur], B.buf["state"][B.cur])
        assert torch.equal(A.buf["slot_k"], B.buf["slot_k"])
        assert torch.equal(A.buf["slot_v"], B.buf["slot_v"])


def test_pageable_host_memory_rejected():
    cfg = synth.WNW_CONFIGS["wnw_tiny"]
    D = WnwDev(cfg, api.WnwParams())
    pageable = np.zeros((4, cfg.capacity, cfg.head_dim), np.uint16)
    L = C.lib()
    st = L.kvc_wnw_recall(ctypes.byref(D.spec.c()), ctypes.byref(D.params.c()),
                          D.buf["state"][0].data_ptr(), pageable.ctypes.data,
                          pageable.ctypes.data, D.buf["slot_k"].data_ptr(),
                          D.buf["slot_v"].data_ptr(), None)
    assert st == C.KVC_ERR_INVALID_ARG
    device = torch.zeros(16, device="cuda")
    st = L.kvc_wnw_recall(ctypes.byref(D.spec.c()), ctypes.byref(D.params.c()),
                          D.buf["state"][0].data_ptr(), device.data_ptr(), device.data_ptr(),
                          D.buf["slot_k"].data_ptr(), D.buf["slot_v"].data_ptr(), None)
    assert st == C.KVC_ERR_INVALID_ARG


def test_voxtral3b_full_size():
    say("[wnw] voxtral3b")
    D = WnwDev(synth.WNW_CONFIGS["wnw_voxtral3b"], api.WnwParams(), fast_host=True)
    for t in range(20):
        D.check_step(t)
    say(f"    {D.n_recalls} blocks recalled, {D.n_releases} released")
    assert D.n_recalls > 0


# ---------------------------------------------------------------------------
# Fixed heads: segment-wise selection
# ---------------------------------------------------------------------------
def _fixed_case(L, H, w, seg, rng):
    sp = api.Spec(n_layers=1, n_kv_heads=H, gqa=2, head_dim=64, seq_lens=[L], retention=[0.5],
                  dtype="bf16", n_window=32)
    prm = api.Params(window=w, base_ratio=0.0)
    rows = [rng.integers(-3, 4, L).astype(np.float32),
            np.round(rng.random(L), 2).astype(np.float32),
            rng.standard_normal(L).astype(np.float32),
            (np.sin(np.arange(L) / 37.0) + 1e-3 * rng.random(L)).astype(np.float32)][:H]
    rows[1][::7] = 0.0
    rows[1][::11] = -0.0
    budgets = np.array([w, L, w + 1 + (L - w) // 3, L - 1][:H], np.int32)
    offsets = np.concatenate([[0], np.cumsum(budgets)]).astype(np.int64)
    sh = torch.from_numpy(np.concatenate(rows)).cuda()
    b = torch.from_numpy(budgets).cuda()
    off = torch.from_numpy(offsets).cuda()
    idx = torch.full((int(offsets[-1]),), -1, dtype=torch.int32, device="cuda")
    api.kvc_wnw_fixed_select(sp, prm, seg, sh, b, off, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for h in range(H):
        want = W.segment_select(rows[h].astype(np.float64), w, int(budgets[h]), seg)
        assert np.array_equal(got[offsets[h]:offsets[h + 1]], want), (L, w, seg, h)


@pytest.mark.parametrize("L", [64, 100, 1000, 3001, 32768])
@pytest.mark.parametrize("seg", [1, 7, 50, 64])
def test_fixed_select_matches_oracle(L, seg):
    say(f"[wnw fixed] L={L} seg={seg}")
    rng = np.random.default_rng(L * 100 + seg)
    _fixed_case(L, 4, 32, seg, rng)
    _fixed_case(L, 4, 0, seg, rng)
