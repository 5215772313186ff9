"""Optional input checks of the prefill entry points (KVC_CHECK_INPUTS=1):
a non-finite query, key or value element, or a negative or non-finite head
score, makes kvc_compress return KVC_ERR_INVALID_ARG without compressing;
valid inputs give the same result as without the checks."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from audio_kv_cache_amd import _lib as C  # noqa: E402
from audio_kv_cache_amd import api, synth  # noqa: E402
from tests.gpu_helpers import Dev  # noqa: E402
import tests.test_gpu_parity as P  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(D, q, k, v, S):
    c = D.cfg
    return api.compress(q, k, v, S, gqa=c.gqa, seq_lens=D.hdr.lengths, retention=D.hdr.retention,
                        alpha=c.alpha, rho=c.rho, window=c.window, base_ratio=c.base_ratio)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_input_checks(monkeypatch, dtype):
    cfg = P.small(dtype=dtype, n_seq=2, lengths=(256, 1000), retention=(0.5, 0.4))
    D = Dev(synth.problem(cfg))
    monkeypatch.delenv("KVC_CHECK_INPUTS", raising=False)
    base = _run(D, D.q, D.k, D.v, D.S)
    monkeypatch.setenv("KVC_CHECK_INPUTS", "1")
    checked = _run(D, D.q, D.k, D.v, D.S)
    torch.cuda.synchronize()
    for key in ("idx", "k_out", "v_out", "budgets", "offsets"):
        assert torch.equal(base[key], checked[key]), key
    bad = float("nan")
    cases = []
    k = D.k.clone(); k[1, 0, 999, 3] = bad; cases.append(("k nan", D.q, k, D.v, D.S))
    v = D.v.clone(); v[0, 1, 5, 0] = float("inf"); cases.append(("v inf", D.q, D.k, v, D.S))
    q = D.q.clone(); q.view(-1)[-1] = -float("inf"); cases.append(("q -inf", q, D.k, D.v, D.S))
    S = D.S.clone(); S.view(-1)[1] = -0.5; cases.append(("S negative", D.q, D.k, D.v, S))
    S2 = D.S.clone(); S2.view(-1)[0] = bad; cases.append(("S nan", D.q, D.k, D.v, S2))
    for name, q_, k_, v_, S_ in cases:
        with pytest.raises(C.KvcError) as e:
            _run(D, q_, k_, v_, S_)
        assert e.value.status == C.KVC_ERR_INVALID_ARG, name


def _stage_inputs(D):
    """Budgets, offsets, smoothed rows and kept positions of a small problem
    from the library's own stage entry points."""
    spec, prm = D.spec, D.params
    rows, ws = api.kvc_plan(spec, prm)
    dev = D.k.device
    b = torch.empty(spec.n_units, dtype=torch.int32, device=dev)
    off = torch.empty(spec.n_units + 1, dtype=torch.int64, device=dev)
    api.kvc_budget(spec, prm, D.S, b, off)
    work = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
    s = torch.empty(spec.score_rows(), dtype=torch.float32, device=dev)
    api.kvc_scores(spec, prm, D.q, D.k, s, work)
    idx = torch.empty(rows, dtype=torch.int32, device=dev)
    api.kvc_select(spec, prm, s, b, off, idx)
    return rows, b, off, s, idx


def test_stage_checks_reject_bad_positions_offsets_and_budgets(monkeypatch):
    cfg = P.small(dtype="bf16", n_seq=2, lengths=(256, 1000), retention=(0.5, 0.4))
    D = Dev(synth.problem(cfg))
    spec, prm = D.spec, D.params
    monkeypatch.delenv("KVC_CHECK_INPUTS", raising=False)
    rows, b, off, s, idx = _stage_inputs(D)
    d = spec.head_dim
    ko = torch.empty((rows, d), dtype=D.k.dtype, device=D.k.device)
    vo = torch.empty_like(ko)
    api.kvc_gather(spec, prm, D.k, D.v, idx, off, ko, vo)
    ref_k = ko.clone()
    monkeypatch.setenv("KVC_CHECK_INPUTS", "1")
    # valid inputs: same result with the checks on
    ko.zero_()
    api.kvc_gather(spec, prm, D.k, D.v, idx, off, ko, vo)
    assert torch.equal(ko, ref_k)
    idx2 = torch.empty_like(idx)
    api.kvc_select(spec, prm, s, b, off, idx2)
    assert torch.equal(idx2, idx)

    def rejects(fn):
        with pytest.raises(C.KvcError) as e:
            fn()
        assert e.value.status == C.KVC_ERR_INVALID_ARG

    L1 = int(D.hdr.lengths[1])
    for bad_pos in (-1, L1, 1 << 30):
        bi = idx.clone()
        bi[-1] = bad_pos                  # last unit belongs to the sequence of length 1000
        rejects(lambda: api.kvc_gather(spec, prm, D.k, D.v, bi, off, ko, vo))
    bo = off.clone(); bo[3] = bo[4] + 1   # a negative segment
    rejects(lambda: api.kvc_gather(spec, prm, D.k, D.v, idx, bo, ko, vo))
    bo = off.clone(); bo[-1] = rows + 64  # past the output rows
    rejects(lambda: api.kvc_gather(spec, prm, D.k, D.v, idx, bo, ko, vo))
    bb = b.clone(); bb[0] += 1            # budgets no longer match the segments
    rejects(lambda: api.kvc_select(spec, prm, s, bb, off, idx2))
    bs = s.clone(); bs[7] = float("nan")
    rejects(lambda: api.kvc_select(spec, prm, bs, b, off, idx2))
