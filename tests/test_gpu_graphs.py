"""HIP graph capture of the library's entry points (torch.cuda.graph drives
hipStreamBeginCapture on the stream the calls are given): a captured
kvc_compress and captured pairs of decode steps (WnW, C3) are replayed
several times, with eager work and synchronisations between the replays,
and every replay is compared bit for bit with the same calls made eagerly.
None of these entry points allocates, synchronises or clears memory with
memset, so their launches are all that the graphs hold.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from audio_kv_cache_amd import api, synth  # noqa: E402
from tests.gpu_helpers import Dev  # noqa: E402
import tests.test_gpu_parity as P  # noqa: E402
from tests.test_gpu_wnw import WnwDev  # noqa: E402
from tests.test_gpu_c3 import C3Dev  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _capture(fn):
    """Warm up fn on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_compress_graph_replays_match_eager():
    say("[graph] compress")
    cfg = P.small(n_seq=2, n_layers=2, n_kv_heads=2, gqa=4, head_dim=128,
                  lengths=(1000, 4096), retention=(0.4, 0.6))
    D = Dev(synth.problem(cfg))
    outs = [api.allocate(D.spec, D.params, "cuda") for _ in range(2)]

    def call(o):
        api.kvc_compress(D.spec, D.params, D.q, D.k, D.v, D.S, o["k_out"], o["v_out"], o["idx"],
                         o["offsets"], o["budgets"], o["workspace"])

    g = _capture(lambda: call(outs[0]))
    for r in range(3):
        for key in ("k_out", "v_out", "idx", "offsets", "budgets"):
            outs[0][key].zero_()
        g.replay()
        call(outs[1])                      # eager work between replays
        torch.cuda.synchronize()
        for key in ("k_out", "v_out", "idx", "offsets", "budgets"):
            assert torch.equal(outs[0][key], outs[1][key]), (r, key)


def test_wnw_step_graph_replays_match_eager():
    say("[graph] wnw")
    cfg, prm = synth.WNW_CONFIGS["wnw_mixed"], api.WnwParams()
    A = WnwDev(cfg, prm)       # eager
    B = WnwDev(cfg, prm)       # graph
    q0 = torch.from_numpy(B.queries(0).view(np.int16)).cuda()
    qa, qb = torch.empty_like(q0), torch.empty_like(q0)
    b = B.buf

    def pair():
        api.kvc_wnw_step(B.spec, prm, qa, B.k, b["state"][0], b["state"][1], B.hk, B.hv,
                         b["slot_k"], b["slot_v"], b["sigma"], b["ws"])
        api.kvc_wnw_step(B.spec, prm, qb, B.k, b["state"][1], b["state"][0], B.hk, B.hv,
                         b["slot_k"], b["slot_v"], b["sigma"], b["ws"])

    # the warm-up inside _capture runs a pair from the initial state: reset after
    qa.copy_(q0)
    qb.copy_(q0)
    g = _capture(pair)
    for st in b["state"]:
        api.kvc_wnw_init(B.spec, prm, st)
    b["slot_k"].zero_()
    b["slot_v"].zero_()
    for r in range(8):
        qa.copy_(torch.from_numpy(B.queries(2 * r).view(np.int16)))
        qb.copy_(torch.from_numpy(B.queries(2 * r + 1).view(np.int16)))
        g.replay()
        A.step(2 * r)
        A.step(2 * r + 1)
        torch.cuda.synchronize()
        assert A.cur == 0
        assert torch.equal(A.buf["state"][0], b["state"][0]), r
        assert torch.equal(A.buf["sigma"], b["sigma"]), r
        assert torch.equal(A.buf["slot_k"], b["slot_k"]), r
        assert torch.equal(A.buf["slot_v"], b["slot_v"]), r


def test_c3_step_graph_replays_match_eager():
    say("[graph] c3")
    cfg = synth.C3_CONFIGS["c3_mixed"]
    A, B = C3Dev(cfg), C3Dev(cfg)
    A.build()
    B.build()
    ob = B.o
    q0 = torch.from_numpy(synth.c3_queries(cfg, 0).view(np.int16)).cuda().view(torch.bfloat16)
    qa, qb = torch.empty_like(q0), torch.empty_like(q0)
    init = ob["state"][0].clone()

    def pair():
        for si, so, q in ((0, 1, qa), (1, 0, qb)):
            api.kvc_c3_step(B.spec, B.params, ob["index"], ob["state"][si], ob["state"][so], q,
                            B.k, B.v, ob["k_out"], ob["v_out"], ob["idx"], ob["step_ws"])

    qa.copy_(q0)
    qb.copy_(q0)
    g = _capture(pair)
    ob["state"][0].copy_(init)
    oa = A.o
    for r in range(6):
        qs = [torch.from_numpy(synth.c3_queries(cfg, 2 * r + i).view(np.int16)).cuda()
              .view(torch.bfloat16) for i in range(2)]
        qa.copy_(qs[0])
        qb.copy_(qs[1])
        g.replay()
        for si, so, q in ((0, 1, qs[0]), (1, 0, qs[1])):
            api.kvc_c3_step(A.spec, A.params, oa["index"], oa["state"][si], oa["state"][so], q,
                            A.k, A.v, oa["k_out"], oa["v_out"], oa["idx"], oa["step_ws"])
        torch.cuda.synchronize()
        VA, VB = A.views(0), B.views(0)
        assert torch.equal(VA.count, VB.count), r
        for u in range(A.U):
            cnt = int(VA.count[u].item())
            assert torch.equal(VA.frontier[u, :cnt], VB.frontier[u, :cnt]), (r, u)
            assert torch.equal(VA.ema[u, :cnt], VB.ema[u, :cnt]), (r, u)
            kept = min(A.n_of(u), A.b_of(u))
            assert torch.equal(oa["idx"][u, :kept], ob["idx"][u, :kept]), (r, u)
            assert torch.equal(oa["k_out"][u, :kept], ob["k_out"][u, :kept]), (r, u)
            assert torch.equal(oa["v_out"][u, :kept], ob["v_out"][u, :kept]), (r, u)
