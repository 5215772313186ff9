"""C-ABI boundary checks that need no GPU: the library loads, exports every
entry point include/kvc.h declares, sizes problems on the host, and rejects
invalid problems before launching anything."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from audio_kv_cache_amd import _lib as C
from audio_kv_cache_amd import api

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def declared_symbols(name):
    text = open(os.path.join(INCLUDE, name)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = C.lib()
    headers = sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h"))
    assert headers == ["kvc.h", "kvc_c3.h", "kvc_voxzip.h", "kvc_wnw.h"]
    assert set(declared_symbols("kvc.h")) == set(C.EXPORTS)
    assert set(declared_symbols("kvc_voxzip.h")) == set(C.VZ_EXPORTS)
    assert set(declared_symbols("kvc_c3.h")) == set(C.C3_EXPORTS)
    assert set(declared_symbols("kvc_wnw.h")) == set(C.WNW_EXPORTS)
    for n in C.EXPORTS + C.VZ_EXPORTS + C.C3_EXPORTS + C.WNW_EXPORTS:
        assert hasattr(L, n), n


def test_status_strings():
    L = C.lib()
    for s in range(6):
        assert L.kvc_status_str(s)
    assert L.kvc_status_str(99) == b"unknown status"
    assert L.kvc_last_hip_error() == 0


def spec(**kw):
    base = dict(n_layers=48, n_kv_heads=4, gqa=8, head_dim=128, seq_lens=[32768],
                retention=0.4, dtype="bf16")
    base.update(kw)
    return api.Spec(**base)


def test_plan_total_rows_same_for_both_budget_pools():
    sp = spec(seq_lens=[8192, 1024], retention=[0.6, 1.0])
    a = api.kvc_plan(sp, api.Params(budget_pool=C.KVC_POOL_SEQUENCE))
    b = api.kvc_plan(sp, api.Params(budget_pool=C.KVC_POOL_LAYER))
    assert a == b


def test_plan_total_rows_closed_form():
    for lens, ret in [([32768], 0.4), ([8192], 0.6), ([1024], 0.6), ([65536], 0.2),
                      ([4096, 32768, 8192], [0.2, 0.55, 1.0])]:
        sp = spec(seq_lens=lens, retention=ret)
        rows, ws = api.kvc_plan(sp, api.Params())
        rets = np.broadcast_to(np.asarray(ret, float), (len(lens),))
        want = sum(48 * 4 * min(math.floor(r * L), L) for L, r in zip(lens, rets))
        assert rows == want
        # score rows + per-unit statistics fit in the workspace
        assert ws >= 4 * 48 * 4 * sum(lens)


def status(sp, prm=None, **ptrs):
    """Call kvc_compress with dummy (never dereferenced) pointers."""
    L = C.lib()
    prm = prm or api.Params()
    fake = ctypes.c_void_p(1 << 20)   # 16-byte and 256-byte aligned, never touched
    args = dict(q=fake, k=fake, v=fake, S=fake, ko=fake, vo=fake, idx=fake, off=fake,
                b=fake, ws=fake)
    args.update(ptrs)
    return L.kvc_compress(ctypes.byref(sp.c()), ctypes.byref(prm.c()), args["q"], args["k"],
                          args["v"], args["S"], args["ko"], args["vo"], args["idx"],
                          args["off"], args["b"], args["ws"], ptrs.get("ws_bytes", 0), None)


def test_invalid_problems_rejected_before_launch():
    assert status(spec(seq_lens=[65537])) == C.KVC_ERR_UNSUPPORTED         # too long
    assert status(spec(seq_lens=[131072])) == C.KVC_ERR_UNSUPPORTED        # too long
    assert status(spec(seq_lens=[32])) == C.KVC_ERR_UNSUPPORTED            # too short
    assert status(spec(head_dim=96)) == C.KVC_ERR_UNSUPPORTED
    assert status(spec(n_window=5)) == C.KVC_ERR_UNSUPPORTED               # G*W = 40, not a multiple of 32
    assert status(spec(gqa=9)) == C.KVC_ERR_UNSUPPORTED                    # G*W = 288 > 256
    assert status(spec(seq_lens=[64], retention=0.5)) == C.KVC_ERR_BUDGET  # w + r > kbar
    assert status(spec(retention=0.0)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(retention=1.5)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), api.Params(alpha=1.5)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), api.Params(rho=0.0)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), api.Params(base_ratio=-0.1)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), api.Params(window=-1)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), api.Params(budget_pool=2)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), api.Params(score_pool=2)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(gqa=16, n_window=16), api.Params(score_pool=1)) == C.KVC_ERR_UNSUPPORTED
    assert status(spec(), q=None) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), ko=ctypes.c_void_p((1 << 20) + 8)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(), ws=ctypes.c_void_p((1 << 20) + 64)) == C.KVC_ERR_INVALID_ARG
    assert status(spec(k_stride=(0, 0, 100))) == C.KVC_ERR_INVALID_ARG    # rows not 16-B aligned
    assert status(spec(k_stride=(0, 0, 64))) == C.KVC_ERR_INVALID_ARG     # stride < head_dim
    assert status(spec()) == C.KVC_ERR_WORKSPACE                           # 0 bytes given
    assert C.lib().kvc_last_hip_error() == 0


def test_lengths_that_are_not_powers_of_two():
    # Bluestein's algorithm takes the transform for these; the workspace
    # grows by the chirp spectrum and two complex rows per unit, and from a
    # Bluestein size M of 32768 on (even L > 16384, odd L > 8192) by the M
    # values of the split transforms per unit.
    for L in (3000, 2047, 32768 - 2, 16383, 100, 16385, 32767, 32770, 49999, 65534, 65535):
        sp = spec(seq_lens=[L], retention=0.9)
        rows, ws = api.kvc_plan(sp, api.Params())
        assert rows == 48 * 4 * math.floor(0.9 * L)
        n_p = L // 2 if L % 2 == 0 else L
        assert ws >= 4 * 48 * 4 * L + 16 * n_p * 48 * 4
        M = 1 << (2 * n_p - 2).bit_length()
        if M >= 32768:
            assert ws >= 4 * 48 * 4 * L + 8 * (M + 2 * n_p) * 48 * 4
    sp = spec(seq_lens=[4096], retention=0.9)
    rows, ws4096 = api.kvc_plan(sp, api.Params())
    assert ws4096 < 4 * 48 * 4 * 4096 + 16 * 2048 * 48 * 4   # powers of two need no scratch


def test_gqa_96_window_queries_is_supported():
    # 3 * 32 = 96 window queries: a multiple of 32, so it is accepted.
    sp = spec(gqa=3)
    assert api.kvc_plan(sp, api.Params())[0] > 0


def test_too_many_sequences_and_units():
    assert status(spec(seq_lens=[64] * 65, retention=0.9,
                       n_layers=1, n_kv_heads=1)) == C.KVC_ERR_UNSUPPORTED
    assert status(spec(n_layers=1025, n_kv_heads=4)) == C.KVC_ERR_UNSUPPORTED


def test_full_retention_plans_every_row():
    sp = spec(seq_lens=[1024], retention=1.0, n_layers=2, n_kv_heads=2)
    assert api.kvc_plan(sp, api.Params())[0] == 4 * 1024


# ---------------------------------------------------------------------------
# include/kvc_voxzip.h
# ---------------------------------------------------------------------------
def vz_spec(**kw):
    base = dict(n_layers=48, n_kv_heads=4, gqa=8, head_dim=128, lens=[8193], budgets=[8192],
                capacity=8200, dtype="bf16")
    base.update(kw)
    return api.VzSpec(**base)


def vz_status(sp, prm=None, ws_bytes=1 << 40):
    L = C.lib()
    prm = prm or api.VzParams()
    fake = ctypes.c_void_p(1 << 20)
    return L.kvc_vz_step(ctypes.byref(sp.c()), ctypes.byref(prm.c()), fake, fake, fake, fake,
                         fake, fake, fake, fake, fake, ws_bytes, None)


def test_vz_plan_closed_form():
    sp = vz_spec(lens=[8193, 100, 4096, 13108], budgets=[8192, 200, 4096, 8192], capacity=13120)
    nl, ws = api.kvc_vz_plan(sp, api.VzParams())
    assert nl.tolist() == [8192, 100, 4096, 8192]
    units = 4 * 48 * 4
    # logits (G per row), chunk statistics, and A before eviction
    assert ws >= units * 13120 * 4 * (8 + 1)


def test_vz_invalid_problems_rejected_before_launch():
    # Every call below fails validation, so the fake pointers are never used;
    # a huge workspace figure makes every shape check reachable.
    assert vz_status(vz_spec(lens=[8201])) == C.KVC_ERR_INVALID_ARG           # n > capacity
    assert vz_status(vz_spec(lens=[0])) == C.KVC_ERR_INVALID_ARG
    assert vz_status(vz_spec(budgets=[0])) == C.KVC_ERR_INVALID_ARG
    assert vz_status(vz_spec(head_dim=96)) == C.KVC_ERR_UNSUPPORTED
    assert vz_status(vz_spec(gqa=33)) == C.KVC_ERR_UNSUPPORTED
    assert vz_status(vz_spec(capacity=70000, lens=[8193])) == C.KVC_ERR_UNSUPPORTED
    assert vz_status(vz_spec(budgets=[4]), api.VzParams(n_sink=4, recent_frac=0.5)) \
        == C.KVC_ERR_BUDGET                                                       # T + M > B
    assert vz_status(vz_spec(), api.VzParams(gamma=-0.1)) == C.KVC_ERR_INVALID_ARG
    assert vz_status(vz_spec(), api.VzParams(recent_frac=1.5)) == C.KVC_ERR_INVALID_ARG
    assert vz_status(vz_spec(), api.VzParams(n_sink=-1)) == C.KVC_ERR_INVALID_ARG
    assert vz_status(vz_spec(), ws_bytes=16) == C.KVC_ERR_WORKSPACE
    assert vz_status(vz_spec(k_stride=(8200 * 128, 100))) == C.KVC_ERR_INVALID_ARG  # row < d


def test_compress_layers_rejects_bad_ranges():
    L = C.lib()
    sp = spec()
    fake = ctypes.c_void_p(1 << 20)
    for lb, le in [(-1, 2), (3, 3), (5, 2), (0, 49)]:
        st = L.kvc_compress_layers(ctypes.byref(sp.c()), ctypes.byref(api.Params().c()), lb, le,
                                   fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                   1 << 40, None)
        assert st == C.KVC_ERR_INVALID_ARG, (lb, le)


# ---------------------------------------------------------------------------
# include/kvc_c3.h
# ---------------------------------------------------------------------------
def c3_spec(**kw):
    base = dict(n_layers=48, n_kv_heads=4, gqa=8, head_dim=128, lens=[32768], budgets=[512],
                capacity=32768)
    base.update(kw)
    return api.C3Spec(**base)


def test_c3_plan_layout():
    sp = c3_spec(lens=[32768, 300, 0], budgets=[512, 512, 512])
    lay = api.kvc_c3_plan(sp, api.C3Params())
    U, NC, CAP, D = sp.n_units, 2 * 32768, 32768, 128
    assert lay.node_cap == NC and lay.kept_cap == 512
    spans = sorted([(lay.start, 4 * U * NC), (lay.size, 4 * U * NC), (lay.left, 4 * U * NC),
                    (lay.parent, 4 * U * NC), (lay.depth, 4 * U * NC), (lay.perm, 4 * U * CAP),
                    (lay.n_nodes, 4 * U), (lay.centroid, 2 * U * NC * D)])
    for (o, n), (o2, _) in zip(spans, spans[1:] + [(lay.index_bytes, 0)]):
        assert o % 256 == 0 and o + n <= o2
    st = sorted([(lay.count, 4 * U), (lay.frontier, 4 * U * CAP), (lay.ema, 8 * U * CAP)])
    for (o, n), (o2, _) in zip(st, st[1:] + [(lay.state_bytes, 0)]):
        assert o % 256 == 0 and o + n <= o2
    assert lay.step_workspace_bytes >= 4 * U * CAP
    # child centroids per position (bf16) dominate the build workspace
    assert lay.build_workspace_bytes >= 2 * U * CAP * D
    # every cache fits its budget: one kept row per cache at least
    assert api.kvc_c3_plan(c3_spec(lens=[0]), api.C3Params()).kept_cap == 1


def c3_status(sp, prm=None, ws_bytes=1 << 40):
    L = C.lib()
    prm = prm or api.C3Params()
    fake = ctypes.c_void_p(1 << 20)
    other = ctypes.c_void_p(1 << 21)
    return L.kvc_c3_step(ctypes.byref(sp.c()), ctypes.byref(prm.c()), fake, fake, other, fake,
                         fake, fake, fake, fake, fake, fake, ws_bytes, None)


def test_c3_invalid_problems_rejected_before_launch():
    assert c3_status(c3_spec(lens=[32769])) == C.KVC_ERR_INVALID_ARG          # n > capacity
    assert c3_status(c3_spec(lens=[-1])) == C.KVC_ERR_INVALID_ARG
    assert c3_status(c3_spec(budgets=[0])) == C.KVC_ERR_INVALID_ARG
    assert c3_status(c3_spec(head_dim=96)) == C.KVC_ERR_UNSUPPORTED
    assert c3_status(c3_spec(gqa=33)) == C.KVC_ERR_UNSUPPORTED
    assert c3_status(c3_spec(capacity=140000, lens=[1000])) == C.KVC_ERR_UNSUPPORTED
    assert c3_status(c3_spec(lens=[1000] * 65, budgets=[10])) == C.KVC_ERR_UNSUPPORTED
    assert c3_status(c3_spec(), api.C3Params(lam=1.5)) == C.KVC_ERR_INVALID_ARG
    assert c3_status(c3_spec(), api.C3Params(r_swaps=9)) == C.KVC_ERR_INVALID_ARG
    assert c3_status(c3_spec(), ws_bytes=16) == C.KVC_ERR_WORKSPACE
    assert c3_status(c3_spec(k_stride=(32768 * 128, 100))) == C.KVC_ERR_INVALID_ARG
    assert c3_status(c3_spec(out_stride=(100 * 128, 128))) == C.KVC_ERR_INVALID_ARG  # < B rows
    # state_in == state_out
    L = C.lib()
    sp = c3_spec()
    fake = ctypes.c_void_p(1 << 20)
    assert L.kvc_c3_step(ctypes.byref(sp.c()), ctypes.byref(api.C3Params().c()), fake, fake,
                         fake, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None) \
        == C.KVC_ERR_INVALID_ARG
    assert L.kvc_c3_build(ctypes.byref(sp.c()), ctypes.byref(api.C3Params().c()), fake, fake,
                          fake, fake, 16, None) == C.KVC_ERR_WORKSPACE


# ---------------------------------------------------------------------------
# include/kvc_wnw.h
# ---------------------------------------------------------------------------
def wnw_spec(**kw):
    prm = api.WnwParams()
    roles = np.full(30 * 8, C.KVC_WNW_TIDAL, np.uint8)
    roles[[12, 45, 77, 101, 160]] = C.KVC_WNW_ANCHOR
    base = dict(n_layers=30, n_kv_heads=8, gqa=4, head_dim=128, lens=[32768], roles=roles,
                capacity=32768, slot_rows=prm.slot_cap * prm.chunk_stride)
    base.update(kw)
    return api.WnwSpec(**base)


def test_wnw_plan_layout():
    prm = api.WnwParams()
    sp = wnw_spec(lens=[32768, 1000, 51])
    lay = api.kvc_wnw_plan(sp, prm)
    assert (lay.n_anchor, lay.n_tidal) == (5, 235)
    assert lay.block_cap == 32768 // 25 + 1 and lay.chunk_cap == lay.block_cap - 1
    assert lay.slot_cap == 3 * 3 * 2
    N = 3
    spans = sorted([(lay.idle, 4 * N * lay.chunk_cap), (lay.slot_of_block, 4 * N * lay.block_cap),
                    (lay.block_of_slot, 4 * N * lay.slot_cap), (lay.selected, 4 * N * 3),
                    (lay.n_recalled, 4 * N), (lay.recalled_block, 4 * N * lay.slot_cap),
                    (lay.recalled_slot, 4 * N * lay.slot_cap)])
    for (o, n), (o2, _) in zip(spans, spans[1:] + [(lay.state_bytes, 0)]):
        assert o % 256 == 0 and o + n <= o2
    # logits of every anchor head dominate the workspace
    assert lay.workspace_bytes >= 4 * N * 5 * 4 * 32768


def wnw_status(sp, prm=None, ws_bytes=1 << 40, same_state=False):
    L = C.lib()
    prm = prm or api.WnwParams()
    fake = ctypes.c_void_p(1 << 20)
    other = ctypes.c_void_p(1 << 21)
    # (every call here must fail validation: nothing may launch on fake pointers)
    if same_state:
        return L.kvc_wnw_update(ctypes.byref(sp.c()), ctypes.byref(prm.c()), fake, fake, fake,
                                None)
    st = L.kvc_wnw_chunk_scores(ctypes.byref(sp.c()), ctypes.byref(prm.c()), fake, fake, fake,
                                fake, ws_bytes, None)
    if st != C.KVC_ERR_WORKSPACE:   # an invalid problem: the update rejects it too
        assert L.kvc_wnw_update(ctypes.byref(sp.c()), ctypes.byref(prm.c()), fake, fake, other,
                                None) == st
    return st


def test_wnw_invalid_problems_rejected_before_launch():
    P = api.WnwParams
    roles = wnw_spec().roles
    assert wnw_status(wnw_spec(lens=[0])) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(lens=[32769])) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(roles=np.where(roles == 1, 0, roles))) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(roles=np.full(240, 3, np.uint8))) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(roles=np.ones(240, np.uint8))) == C.KVC_ERR_UNSUPPORTED  # 240 anchors
    assert wnw_status(wnw_spec(), P(chunk_len=60)) == C.KVC_ERR_INVALID_ARG   # not a multiple
    assert wnw_status(wnw_spec(), P(chunk_len=10)) == C.KVC_ERR_INVALID_ARG   # shorter than S
    assert wnw_status(wnw_spec(), P(chunk_len=225)) == C.KVC_ERR_UNSUPPORTED  # m = 9
    assert wnw_status(wnw_spec(), P(top_chunks=0)) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(), P(top_chunks=9)) == C.KVC_ERR_UNSUPPORTED
    assert wnw_status(wnw_spec(), P(release_after=9)) == C.KVC_ERR_UNSUPPORTED
    assert wnw_status(wnw_spec(head_dim=96)) == C.KVC_ERR_UNSUPPORTED
    assert wnw_status(wnw_spec(gqa=33)) == C.KVC_ERR_UNSUPPORTED
    assert wnw_status(wnw_spec(capacity=140000, lens=[1000])) == C.KVC_ERR_UNSUPPORTED
    assert wnw_status(wnw_spec(lens=[1000] * 65)) == C.KVC_ERR_UNSUPPORTED
    assert wnw_status(wnw_spec(k_stride=(32768 * 128, 100))) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(host_stride=(1000 * 128, 128))) == C.KVC_ERR_INVALID_ARG
    assert wnw_status(wnw_spec(slot_rows=100)) == C.KVC_ERR_INVALID_ARG       # < 18 blocks
    assert wnw_status(wnw_spec(), ws_bytes=16) == C.KVC_ERR_WORKSPACE
    assert wnw_status(wnw_spec(), same_state=True) == C.KVC_ERR_INVALID_ARG


def test_wnw_fixed_select_rejects_segment_lengths():
    L = C.lib()
    sp = api.Spec(n_layers=2, n_kv_heads=2, gqa=2, head_dim=64, seq_lens=[256], retention=[0.5],
                  dtype="bf16")
    fake = ctypes.c_void_p(1 << 20)
    for seg in (0, 65):
        assert L.kvc_wnw_fixed_select(ctypes.byref(sp.c()), ctypes.byref(api.Params().c()), seg,
                                      fake, fake, fake, fake, None) == C.KVC_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# The torch wrapper's own checks: every rejection happens before any pointer
# reaches the library (CPU tensors, so no GPU is touched either way).
# ---------------------------------------------------------------------------
def _wrapper_inputs(NL=2, H=2, G=2, W=32, d=64, T=256, dt=None):
    import torch
    dt = dt or torch.bfloat16
    q = torch.zeros((1, NL, H * G, W, d), dtype=dt)
    k = torch.zeros((NL, H, T, d), dtype=dt)
    v = torch.zeros((NL, H, T, d), dtype=dt)
    S = torch.zeros((NL, H), dtype=torch.float32)
    return q, k, v, S


@pytest.mark.parametrize("case", [
    "f16", "mixed", "q_dtype", "kv_shape", "k_stride", "v_stride", "too_long", "q_count",
    "q_strided", "q_last_dim", "s_dtype", "s_shape", "s_strided"])
def test_compress_wrapper_rejects_mismatched_tensors(case):
    import torch
    q, k, v, S = _wrapper_inputs()
    lens = [256]
    msg = None
    if case == "f16":
        q, k, v = q.half(), k.half(), v.half()
        msg = "bfloat16 or float32"
    elif case == "mixed":
        v = v.float()
        msg = "share one dtype"
    elif case == "q_dtype":
        q = q.float()
        msg = "share one dtype"
    elif case == "kv_shape":
        v = v[:, :, :128]
        msg = "n_layers, n_kv_heads, T, head_dim"
    elif case == "k_stride":
        k = torch.zeros((2, 2, 64, 256), dtype=torch.bfloat16).transpose(2, 3)
        msg = "head_dim contiguous"
    elif case == "v_stride":
        v = torch.zeros((2, 2, 64, 256), dtype=torch.bfloat16).transpose(2, 3)
        msg = "head_dim contiguous"
    elif case == "too_long":
        lens = [200, 100]
        msg = "sum(seq_lens)"
    elif case == "q_count":
        q = q[:, :1]
        msg = "elements"
    elif case == "q_strided":
        q = torch.zeros((1, 2, 4, 64, 32), dtype=torch.bfloat16).transpose(3, 4)
        msg = "contiguous"
    elif case == "q_last_dim":
        q = torch.zeros((1, 2, 4, 64, 32), dtype=torch.bfloat16)
        msg = "head_dim"
    elif case == "s_dtype":
        S = S.double()
        msg = "head_scores"
    elif case == "s_shape":
        S = torch.zeros((2, 3), dtype=torch.float32)
        msg = "head_scores"
    elif case == "s_strided":
        S = torch.zeros((2, 4), dtype=torch.float32)[:, ::2]
        msg = "head_scores"
    with pytest.raises(ValueError, match=re.escape(msg)):
        api.compress(q, k, v, S, gqa=2, seq_lens=lens, retention=0.6)


def test_compress_wrapper_accepts_consistent_cpu_tensors_up_to_the_device_check():
    # Well-formed tensors pass every layout check and then fail only because
    # they are not in GPU memory.
    q, k, v, S = _wrapper_inputs()
    with pytest.raises(ValueError, match="GPU memory"):
        api.compress(q, k, v, S, gqa=2, seq_lens=[256], retention=0.6)


def test_noalloc_entry_point_rejects_before_touching_the_device():
    # A problem whose workspace exceeds the static array, and null pointers,
    # are refused on the host (dummy pointers are never dereferenced).
    L = C.lib()
    big = spec(seq_lens=[65536, 65536], retention=0.2)   # about 120 MiB of workspace
    prm = api.Params()
    assert api.kvc_plan(big, prm)[1] > C.KVC_NOALLOC_MAX_WORKSPACE
    fake = ctypes.c_void_p(1 << 20)
    args = [fake] * 9
    assert L.kvc_compress_noalloc(ctypes.byref(big.c()), ctypes.byref(prm.c()), *args,
                                  None) == C.KVC_ERR_WORKSPACE
    ok = spec(seq_lens=[8192], retention=0.6, n_layers=28, gqa=7)
    assert api.kvc_plan(ok, prm)[1] <= C.KVC_NOALLOC_MAX_WORKSPACE
    nulls = [fake] * 8 + [None]
    assert L.kvc_compress_noalloc(ctypes.byref(ok.c()), ctypes.byref(prm.c()), *nulls,
                                  None) == C.KVC_ERR_INVALID_ARG
