"""GPU parity of every step against the fp64 oracle, through the C ABI.

Small configurations are checked element by element; the full-size
configurations (the ones bench.py times) on sampled units the oracle
computes one by one.  Criteria are those in gpu_helpers.
"""
import dataclasses
import json
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from audio_kv_cache_amd import api, synth  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests.gpu_helpers import (TOL, Dev, check_kept_sets, check_smoothed_row,  # noqa: E402
                               rel_err)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


_cache = {}


def dev(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _cache:
        cfg = synth.CONFIGS[name]
        if kw:
            cfg = dataclasses.replace(cfg, **kw)
        say(f"[gen] {name} {kw}")
        _cache.clear()   # keep one full-size problem resident at a time
        _cache[key] = Dev(synth.problem(cfg))
    return _cache[key]


def small(name="t", **kw):
    base = dict(name=name, index=50, n_seq=1, n_layers=2, n_kv_heads=2, gqa=2, head_dim=64,
                dtype="bf16", lengths=(256,), retention=(0.5,))
    base.update(kw)
    return synth.Config(**base)


# ---------------------------------------------------------------------------
# Step 3: budgets (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "qwen7b", "omni30b", "ragged", "long64k"])
def test_budget_bitexact_configs(name):
    say(f"[budget] {name}")
    cfg = synth.CONFIGS[name]
    hdr = synth.header(cfg)
    # budgets need no K/V: a header-only device problem
    spec = api.Spec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                    head_dim=cfg.head_dim, seq_lens=hdr.lengths, retention=hdr.retention,
                    dtype=cfg.dtype, n_window=cfg.n_window)
    prm = api.Params(cfg.alpha, cfg.rho, cfg.window, cfg.base_ratio)
    S = torch.from_numpy(hdr.head_scores).cuda()
    b = torch.empty(spec.n_units, dtype=torch.int32, device="cuda")
    off = torch.empty(spec.n_units + 1, dtype=torch.int64, device="cuda")
    api.kvc_budget(spec, prm, S, b, off)
    torch.cuda.synchronize()
    want = np.concatenate([O.budget(hdr.head_scores, int(L), float(r), cfg.base_ratio, cfg.window)
                           for L, r in zip(hdr.lengths, hdr.retention)])
    assert np.array_equal(b.cpu().numpy(), want)
    assert np.array_equal(off.cpu().numpy(), np.concatenate([[0], np.cumsum(want)]))
    assert int(off[-1]) == api.kvc_plan(spec, prm)[0]


@pytest.mark.parametrize("name", ["tiny", "qwen7b", "omni30b", "ragged", "long64k"])
def test_budget_bitexact_layer_pool(name):
    say(f"[budget] layer pool {name}")
    cfg = dataclasses.replace(synth.CONFIGS[name], budget_pool=1)
    hdr = synth.header(cfg)
    spec = api.Spec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                    head_dim=cfg.head_dim, seq_lens=hdr.lengths, retention=hdr.retention,
                    dtype=cfg.dtype, n_window=cfg.n_window)
    prm = api.Params(cfg.alpha, cfg.rho, cfg.window, cfg.base_ratio, budget_pool=1)
    S = torch.from_numpy(hdr.head_scores).cuda()
    b = torch.empty(spec.n_units, dtype=torch.int32, device="cuda")
    off = torch.empty(spec.n_units + 1, dtype=torch.int64, device="cuda")
    api.kvc_budget(spec, prm, S, b, off)
    torch.cuda.synchronize()
    want, want_off = O.problem_budgets(synth.Problem(hdr, None, None, None), budget_pool=1)
    assert np.array_equal(b.cpu().numpy(), want)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert int(off[-1]) == api.kvc_plan(spec, prm)[0]


def _budget_gpu(S, L, ret, base, w):
    S = np.asarray(S, np.float32).reshape(1, -1)
    spec = api.Spec(n_layers=1, n_kv_heads=S.shape[1], gqa=1, head_dim=64, seq_lens=[L],
                    retention=ret, dtype="f32", n_window=32)
    prm = api.Params(0.5, 0.7, w, base)
    St = torch.from_numpy(S).cuda()
    b = torch.empty(S.shape[1], dtype=torch.int32, device="cuda")
    off = torch.empty(S.shape[1] + 1, dtype=torch.int64, device="cuda")
    api.kvc_budget(spec, prm, St, b, off)
    torch.cuda.synchronize()
    return b.cpu().numpy()


def test_budget_bitexact_hand_cases_and_random():
    here = os.path.dirname(__file__)
    gold = json.load(open(os.path.join(here, "golden", "budget_hand.json")))
    assert len(gold["cases"]) == 7
    for c in gold["cases"]:
        say(f"[budget] hand: {c['name']}")
        got = _budget_gpu(c["S"], c["L"], c["retention"], c["base_ratio"], c["window"])
        assert got.tolist() == c["budgets"]
    rng = np.random.default_rng(5)
    for it in range(60):
        n = int(rng.integers(1, 300))
        L = int(rng.choice([64, 256, 1024, 8192, 32768, 65536]))
        ret = float(rng.uniform(0.05, 1.0))
        base = float(rng.choice([0.0, 0.3, 0.5]))
        kind = it % 3
        S = (rng.uniform(0, 1, n) if kind == 0 else
             np.where(rng.random(n) < 0.18, rng.uniform(0.6, 1, n), rng.uniform(0, 0.2, n))
             if kind == 1 else rng.integers(0, 3, n).astype(float))
        if O.budget_rc(S, L, ret, base, 32) != 0:
            continue
        assert np.array_equal(_budget_gpu(S, L, ret, base, 32), O.budget(S, L, ret, base, 32))
    # Scores spread over about 80 binades: partial sums are no longer exact
    # in fp64, so the kernel's rounds take the sequential sum in head order.
    for it in range(12):
        n = int(rng.integers(2, 400))
        S = (rng.uniform(0.5, 1.0, n) * np.exp2(-rng.integers(0, 80, n))).astype(np.float32)
        S[rng.random(n) < 0.1] = 0.0
        L = int(rng.choice([1024, 8192, 32768]))
        ret = float(rng.uniform(0.3, 0.9))
        if O.budget_rc(S, L, ret, 0.5, 32) != 0:
            continue
        assert np.array_equal(_budget_gpu(S, L, ret, 0.5, 32), O.budget(S, L, ret, 0.5, 32)), it


# ---------------------------------------------------------------------------
# Step 5: gather (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d,many", [("bf16", 128, False), ("bf16", 64, False), ("f32", 64, False),
                                           ("f32", 128, False), ("bf16", 128, True)])
def test_gather_bitexact(dtype, d, many):
    """many: 1152 units, more than the gather stages in LDS (it then looks up
    each row's unit in global memory)."""
    say(f"[gather] {dtype} d={d} many={many}")
    if many:
        cfg = small(dtype=dtype, head_dim=d, n_seq=3, n_layers=24, n_kv_heads=16, lengths=(64, 96, 128),
                    retention=(0.5, 0.7, 0.4), base_ratio=0.0)
    else:
        cfg = small(dtype=dtype, head_dim=d, n_seq=3, lengths=(256, 1024, 128), retention=(0.5, 0.3, 0.9),
                    base_ratio=0.0)
    D = Dev(synth.problem(cfg))
    b, off = D.budget()
    rng = np.random.default_rng(1)
    idx = np.empty(int(off[-1]), np.int32)
    for (i, l, h) in D.units():
        u = D.uindex(i, l, h)
        L = int(D.hdr.lengths[i])
        idx[off[u]:off[u + 1]] = np.sort(rng.choice(L, size=int(b[u]), replace=False))
    ko, vo = D.gather(idx, off)
    for (i, l, h) in D.units():
        u = D.uindex(i, l, h)
        _, ku, vu = O.unit_inputs(D.prob, i, l, h)
        sel = idx[off[u]:off[u + 1]]
        assert np.array_equal(ko[off[u]:off[u + 1]], ku[sel])
        assert np.array_equal(vo[off[u]:off[u + 1]], vu[sel])


# ---------------------------------------------------------------------------
# Step 4: selection on identical scores (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("L", [64, 128, 1024, 4096, 16384, 32768, 65536])
def test_select_bitexact_with_ties(L):
    say(f"[select] L={L}")
    H = 4
    cfg = small(n_layers=1, n_kv_heads=H, lengths=(L,), retention=(0.5,), base_ratio=0.0)
    D = Dev(synth.problem(cfg))
    rng = np.random.default_rng(L)
    w = cfg.window
    rows = []
    # ties, negative values, signed zeros, and a smooth row
    rows.append(rng.integers(-3, 4, L).astype(np.float32))
    r = rng.standard_normal(L).astype(np.float32); r[::7] = 0.0; r[::11] = -0.0
    rows.append(r)
    rows.append(np.round(rng.random(L), 2).astype(np.float32))
    rows.append((np.sin(np.arange(L) / 37.0) + 1e-3 * rng.random(L)).astype(np.float32))
    sh = np.concatenate(rows)
    # budgets from k = 0 to k = L - w
    budgets = np.array([w, L, w + 1 + (L - w) // 3, L - 1], np.int32)
    offsets = np.concatenate([[0], np.cumsum(budgets)]).astype(np.int64)
    idx = D.select(sh, budgets, offsets)
    for h in range(H):
        want = O.select(rows[h].astype(np.float64), w, int(budgets[h]))
        got = idx[offsets[h]:offsets[h + 1]]
        assert np.array_equal(got, want), (h, int(budgets[h]))


# ---------------------------------------------------------------------------
# Step 2: smoothing on identical rows
# ---------------------------------------------------------------------------
def _sss_rows(L, n, rng):
    j = np.arange(L)
    rows = []
    sink = np.exp(-np.arange(L) / 3.0); sink /= sink.sum()
    rows.append(0.4 * sink + 0.6 * (1 + 0.3 * np.sin(2 * np.pi * j / 200)) / L)     # sink + drift
    rows.append((1 + 0.5 * np.cos(2 * np.pi * 5 * j / L) + 0.05 * rng.random(L)) / L)  # no sink
    rows.append(rng.random(L) ** 6)                                                  # spiky
    rows.append(np.full(L, 1.0 / 1024))                                              # constant
    return [r.astype(np.float32) for r in rows[:n]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [64, 256, 1024, 2048, 8192, 16384, 32768, 65536])
def test_smooth_matches_oracle(L, dtype):
    say(f"[smooth] L={L} {dtype}")
    for alpha, rho in [(0.5, 0.7), (0.6, 0.7), (1.0, 0.95), (0.3, 0.2)]:
        cfg = small(n_layers=1, n_kv_heads=4, lengths=(L,), dtype=dtype, alpha=alpha, rho=rho,
                    retention=(0.9,), base_ratio=0.0)
        D = Dev(synth.problem(cfg))
        rows = _sss_rows(L, 4, np.random.default_rng(L))
        sh, ks = D.smooth(np.concatenate(rows))
        for h in range(4):
            check_smoothed_row(rows[h], sh[h * L:(h + 1) * L], int(ks[h]), alpha, rho, dtype)
            if h == 3:   # constant row: k* = 0 and the row passes through
                assert int(ks[h]) == 0
                assert rel_err(sh[3 * L:4 * L], rows[3]) <= 1e-6


def test_smooth_alpha_zero_is_identity_bitexact():
    L = 4096
    cfg = small(n_layers=1, n_kv_heads=4, lengths=(L,), alpha=0.0, retention=(0.9,), base_ratio=0.0)
    D = Dev(synth.problem(cfg))
    rows = np.concatenate(_sss_rows(L, 4, np.random.default_rng(3)))
    sh, _ = D.smooth(rows)
    assert np.array_equal(sh, rows)


# ---------------------------------------------------------------------------
# Step 1: scores
# ---------------------------------------------------------------------------
def _check_scores(D, units):
    s = D.scores()
    worst = 0.0
    for (i, l, h) in units:
        qu, ku, _ = O.unit_inputs(D.prob, i, l, h)
        q = O.widen(qu, D.dtype).reshape(-1, D.cfg.head_dim)
        if D.cfg.score_pool == 1:
            ref = O.scores_maxpool(q, O.widen(ku, D.dtype), D.cfg.n_window)
        else:
            ref = O.scores(q, O.widen(ku, D.dtype))
        err = rel_err(D.row(s, i, l, h), ref)
        worst = max(worst, err)
        assert err <= TOL[D.dtype], ((i, l, h), err)
    say(f"    worst row error {worst:.2e}")
    return s


def test_scores_tiny_all_units():
    say("[scores] tiny")
    D = dev("tiny")
    _check_scores(D, D.units())


@pytest.mark.parametrize("d,gqa", [(64, 2), (128, 1), (128, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scores_small_shapes(dtype, d, gqa):
    say(f"[scores] small {dtype} d={d} gqa={gqa}")
    cfg = small(dtype=dtype, head_dim=d, gqa=gqa, n_seq=2, lengths=(2048, 64), retention=(0.5, 0.9),
                base_ratio=0.0)
    D = Dev(synth.problem(cfg))
    _check_scores(D, D.units())


def test_scores_qwen7b_sampled():
    say("[scores] qwen7b")
    D = dev("qwen7b")
    _check_scores(D, [(0, 0, 0), (0, 13, 2), (0, 27, 3)])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scores_two_pass_entry_points(dtype):
    say(f"[scores] stats + pool entry points, {dtype}")
    cfg = small(dtype=dtype, n_seq=2, lengths=(4096, 1024), retention=(0.5, 0.5), base_ratio=0.0)
    D = Dev(synth.problem(cfg))
    s2 = D.scores_two_pass()
    assert np.array_equal(s2, D.scores())
    for (i, l, h) in D.units():
        qu, ku, _ = O.unit_inputs(D.prob, i, l, h)
        ref = O.scores(O.widen(qu, D.dtype).reshape(-1, D.cfg.head_dim), O.widen(ku, D.dtype))
        assert rel_err(D.row(s2, i, l, h), ref) <= TOL[D.dtype]


@pytest.mark.parametrize("dtype,d,gqa,W", [("bf16", 128, 8, 32), ("bf16", 64, 7, 32),
                                           ("bf16", 128, 1, 32), ("bf16", 128, 2, 64),
                                           ("f32", 64, 2, 32), ("f32", 128, 2, 64)])
def test_scores_maxpool(dtype, d, gqa, W):
    say(f"[scores] max over heads {dtype} d={d} G={gqa} W={W}")
    cfg = small(dtype=dtype, head_dim=d, gqa=gqa, n_window=W, n_seq=2, lengths=(2048, 128),
                retention=(0.5, 0.9), base_ratio=0.0, score_pool=1)
    D = Dev(synth.problem(cfg))
    _check_scores(D, D.units())


@pytest.mark.parametrize("case", ["late_spike", "early_spike"])
def test_scores_reference_overflow_and_underflow(case):
    # The bf16 statistics pass sums exp2 against a reference taken from each
    # tile's first 32 keys.  late_spike: a key far past them whose logit
    # exceeds the reference by far more than the fp32 exponent range (the
    # pass must fall back to the exact online maximum); early_spike: the
    # first keys dominate and every later term underflows against them.
    say(f"[scores] reference {case}")
    cfg = small(dtype="bf16", head_dim=128, gqa=8, n_seq=1, lengths=(2048,), retention=(0.5,),
                base_ratio=0.0, n_layers=1, n_kv_heads=1)
    prob = synth.problem(cfg)
    qm = synth.bf16_bits_to_f32(prob.q[0, 0].reshape(-1, 128)).mean(axis=0)
    k = synth.bf16_bits_to_f32(prob.k[0, 0]).copy()
    if case == "late_spike":
        k[:64] = 0.0
        k[1500] = 8.0 * qm / np.linalg.norm(qm) * 40.0
    else:
        k[:32] = 8.0 * qm / np.linalg.norm(qm) * 40.0
        k[32:] *= 0.05
    prob.k[0, 0] = synth.f32_to_bf16_bits(k)
    D = Dev(prob)
    _check_scores(D, D.units())


@pytest.mark.parametrize("name,units", [("omni30b", [(0, 0, 0), (0, 31, 2)]),
                                        ("long64k", [(0, 47, 3)])])
def test_scores_and_smoothing_full_size_sampled(name, units):
    # The launch configuration the benchmark times (every unit of the
    # problem in one launch per pass): s element by element against the
    # oracle on sampled units, then s_hat and k* of those rows.
    say(f"[scores+smooth] {name} {units}")
    D = dev(name)
    s = _check_scores(D, units)
    sh, ks = D.smooth(s)
    for (i, l, h) in units:
        u = D.uindex(i, l, h)
        err, _ = check_smoothed_row(D.row(s, i, l, h), D.row(sh, i, l, h), int(ks[u]),
                                    D.cfg.alpha, D.cfg.rho, D.dtype)
        say(f"    unit {(i, l, h)}: k* {int(ks[u])}, s_hat error {err:.2e}")


def test_scores_no_sink_variant():
    say("[scores] qwen7b-shaped, no sink")
    cfg = dataclasses.replace(synth.CONFIGS["qwen7b"], n_layers=2, sink_beta=0.0)
    D = Dev(synth.problem(cfg))
    _check_scores(D, D.units())


# ---------------------------------------------------------------------------
# End to end
# ---------------------------------------------------------------------------
def _check_e2e(D, units):
    o = D.compress()
    b_ref, off_ref = O.problem_budgets(D.prob)
    b = o["budgets"].cpu().numpy()
    off = o["offsets"].cpu().numpy()
    assert np.array_equal(b, b_ref) and np.array_equal(off, off_ref)
    idx = o["idx"].cpu().numpy()
    ko = o["k_out"]
    vo = o["v_out"]
    ndiff = 0
    for (i, l, h) in units:
        u = D.uindex(i, l, h)
        qu, ku, vu = O.unit_inputs(D.prob, i, l, h)
        r = O.unit_compress(qu, ku, D.dtype, int(b[u]), D.cfg.alpha, D.cfg.rho, D.cfg.window,
                            D.cfg.score_pool)
        got = idx[off[u]:off[u + 1]]
        ndiff += check_kept_sets(got, r["kept"], r["s_hat"], int(b[u]), D.cfg.window, D.dtype)
        kon = ko[off[u]:off[u + 1]]
        von = vo[off[u]:off[u + 1]]
        if D.dtype == "bf16":
            kon, von = kon.view(torch.int16), von.view(torch.int16)
        kon = kon.cpu().numpy().view(ku.dtype)
        von = von.cpu().numpy().view(vu.dtype)
        assert np.array_equal(kon, ku[got]) and np.array_equal(von, vu[got])
    say(f"    units {len(units)}, near-threshold set differences {ndiff}")
    return o


def test_compress_tiny():
    say("[e2e] tiny")
    D = dev("tiny")
    _check_e2e(D, D.units())


def test_compress_qwen7b_sampled():
    say("[e2e] qwen7b")
    D = dev("qwen7b")
    _check_e2e(D, [(0, 0, 0), (0, 7, 1), (0, 20, 3)])


def test_compress_ragged_sampled():
    say("[e2e] ragged")
    D = dev("ragged")
    units = []
    seen = set()
    for i, L in enumerate(D.hdr.lengths):
        if int(L) not in seen:
            seen.add(int(L))
            units.append((i, 3, 1))
    _check_e2e(D, units)


def test_compress_omni30b_sampled():
    say("[e2e] omni30b")
    D = dev("omni30b")
    _check_e2e(D, [(0, 0, 0), (0, 31, 2)])


def test_compress_qwen7b_layer_pool_sampled():
    say("[e2e] qwen7b, one budget pool per layer")
    D = dev("qwen7b", budget_pool=1)
    _check_e2e(D, [(0, 0, 0), (0, 13, 2), (0, 27, 3)])


def test_compress_qwen7b_maxpool_sampled():
    say("[e2e] qwen7b, max over query heads")
    D = dev("qwen7b", score_pool=1)
    _check_e2e(D, [(0, 0, 0), (0, 13, 2), (0, 27, 3)])


def test_compress_long64k_sampled():
    say("[e2e] long64k")
    D = dev("long64k")
    _check_e2e(D, [(0, 47, 3)])


def test_compress_full_retention_identity():
    say("[e2e] retention 1")
    cfg = small(retention=(1.0,), lengths=(512,))
    D = Dev(synth.problem(cfg))
    o = D.compress()
    idx = o["idx"].cpu().numpy()
    assert np.array_equal(idx, np.tile(np.arange(512), 4))
    assert torch.equal(o["k_out"].view(4, 512, -1), D.k.reshape(4, 512, -1))


@pytest.mark.parametrize("case,kw", [
    # shortest length, no local window (every kept row comes from the top-k)
    ("L64_w0", dict(lengths=(64,), window=0, retention=(0.5,))),
    # mean budget equal to the window with no base share: the pool is empty
    # and every unit keeps exactly its last 32 positions
    ("budget_is_window", dict(lengths=(64,), window=32, retention=(0.5,), base_ratio=0.0)),
    # two odd lengths, one query head per KV head, no window; some heads'
    # budgets reach L (every position kept)
    ("odd_w0_g1", dict(n_seq=2, lengths=(65, 97), window=0, retention=(0.3, 0.7), head_dim=128,
                       gqa=1)),
    # a one-position window, retention 0.9 beside 0.05 (budgets of 3 to 5 rows)
    ("w1_extremes", dict(n_seq=2, lengths=(64, 127), window=1, retention=(0.9, 0.05),
                         base_ratio=0.0)),
])
def test_compress_edge_shapes(case, kw):
    say(f"[e2e] edge {case}")
    cfg = small(name="edge", n_layers=3, n_kv_heads=2, **kw)
    D = Dev(synth.problem(cfg))
    o = _check_e2e(D, D.units())
    if case == "budget_is_window":
        assert np.array_equal(o["idx"].cpu().numpy(), np.tile(np.arange(32, 64), 6))


def test_compress_deterministic():
    say("[e2e] determinism")
    D = dev("qwen7b")
    a = D.compress()
    b = D.compress()
    for key in ("idx", "k_out", "v_out", "budgets", "offsets"):
        assert torch.equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# Streaming prefill: layer-range calls reproduce the whole-model call
# ---------------------------------------------------------------------------
def test_compress_independent_of_launch_order_and_grid():
    # Every layer of omni30b compressed by its own call, in a shuffled order:
    # each call's launches hold one layer's units (a different number of
    # workgroups and so a different mapping of score tiles onto the XCDs and
    # CUs), and units run in another order.  The outputs must equal the
    # whole-model call's bit for bit.
    say("[e2e] omni30b, one call per layer in shuffled order")
    D = dev("omni30b")
    whole = D.compress()
    out = api.allocate(D.spec, D.params, "cuda")
    for t in ("k_out", "v_out"):
        out[t].zero_()
    out["idx"].fill_(-1)
    order = np.random.default_rng(7).permutation(D.cfg.n_layers)
    for l in order.tolist():
        api.kvc_compress_layers(D.spec, D.params, l, l + 1, D.q[:, l:l + 1].contiguous(),
                                D.k[l:l + 1], D.v[l:l + 1], D.S, out["k_out"], out["v_out"],
                                out["idx"], out["offsets"], out["budgets"], out["workspace"])
    torch.cuda.synchronize()
    for key in ("budgets", "offsets", "idx"):
        assert torch.equal(out[key], whole[key]), key
    for key in ("k_out", "v_out"):
        assert torch.equal(out[key].view(torch.int16), whole[key].view(torch.int16)), key


@pytest.mark.parametrize("name,ranges", [("qwen7b", [(0, 1), (1, 3), (3, 4)]),
                                         ("ragged", [(0, 2), (2, 3)])])
def test_compress_layers_equals_whole_call(name, ranges):
    say(f"[e2e] layer ranges {name} {ranges}")
    NL = ranges[-1][1]
    cfg = dataclasses.replace(synth.CONFIGS[name], n_layers=NL)
    if name == "ragged":
        cfg = dataclasses.replace(cfg, n_seq=3)
    D = Dev(synth.problem(cfg))
    whole = D.compress()
    out = api.allocate(D.spec, D.params, "cuda")
    for t in ("k_out", "v_out"):
        out[t].zero_()
    out["idx"].fill_(-1)
    for lb, le in ranges:
        # each range's inputs in buffers of their own, as a streaming caller has them
        q = D.q[:, lb:le].contiguous()
        k = D.k[lb:le].contiguous()
        v = D.v[lb:le].contiguous()
        api.kvc_compress_layers(D.spec, D.params, lb, le, q, k, v, D.S, out["k_out"],
                                out["v_out"], out["idx"], out["offsets"], out["budgets"],
                                out["workspace"])
    torch.cuda.synchronize()
    for key in ("budgets", "offsets", "idx"):
        assert torch.equal(out[key], whole[key]), key
    for key in ("k_out", "v_out"):
        assert torch.equal(out[key].view(torch.int16) if D.dtype == "bf16" else out[key],
                           whole[key].view(torch.int16) if D.dtype == "bf16" else whole[key]), key
