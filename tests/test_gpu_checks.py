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
