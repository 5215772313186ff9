"""kvc_compress_noalloc (workspace in the library's static per-device array)
against kvc_compress (a caller-supplied workspace), through the C ABI: the
same kernels on the same inputs, so the outputs must be identical bit for
bit.  Two calls in a row on one device, the second on a smaller problem (the
array keeps the first call's contents), and a problem over the limit
rejected before any work is enqueued."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from audio_kv_cache_amd import _lib as C  # noqa: E402
from audio_kv_cache_amd import api, synth  # noqa: E402
from tests.gpu_helpers import Dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _noalloc(D):
    """Outputs of kvc_compress_noalloc, pre-filled with garbage so that every
    element must be written."""
    rows, _ = api.kvc_plan(D.spec, D.params)
    d = D.spec.head_dim
    dev = D.k.device
    o = dict(k_out=torch.full((rows, d), 7, dtype=D.k.dtype, device=dev),
             v_out=torch.full((rows, d), 7, dtype=D.k.dtype, device=dev),
             idx=torch.full((rows,), -5, dtype=torch.int32, device=dev),
             offsets=torch.full((D.spec.n_units + 1,), -5, dtype=torch.int64, device=dev),
             budgets=torch.full((D.spec.n_units,), -5, dtype=torch.int32, device=dev))
    api.kvc_compress_noalloc(D.spec, D.params, D.q, D.k, D.v, D.S, o["k_out"], o["v_out"],
                             o["idx"], o["offsets"], o["budgets"])
    torch.cuda.synchronize()
    return o


def _same(a, b, dtype):
    for key in ("budgets", "offsets", "idx"):
        assert torch.equal(a[key], b[key]), key
    for key in ("k_out", "v_out"):
        x, y = a[key], b[key]
        if dtype == "bf16":
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), key


def test_noalloc_equals_compress_on_two_calls_in_a_row():
    # First call: the 48-layer, 4-KV-head, L = 32768 problem (about 36 MiB
    # of workspace); second: three short sequences of lengths that are not
    # powers of two (a smaller workspace with a different layout, including
    # the Bluestein scratch), on the same device's array.
    big = Dev(synth.problem(synth.CONFIGS["omni30b"]))
    ref_big = big.compress()
    got_big = _noalloc(big)
    _same(got_big, ref_big, big.dtype)
    del big, ref_big, got_big
    small_cfg = synth.CONFIGS["ragged_npot"]
    small = Dev(synth.problem(small_cfg))
    ref_small = small.compress()
    got_small = _noalloc(small)
    _same(got_small, ref_small, small.dtype)
    # and again on the first, smaller, problem after the second
    tiny = Dev(synth.problem(synth.CONFIGS["tiny"]))
    _same(_noalloc(tiny), tiny.compress(), tiny.dtype)


def test_noalloc_rejects_problems_over_the_limit():
    cfg = synth.CONFIGS["long64k"]            # two of them: about 120 MiB of workspace
    hdr = synth.header(cfg)
    spec = api.Spec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                    head_dim=cfg.head_dim, seq_lens=list(hdr.lengths) * 2,
                    retention=list(hdr.retention) * 2,
                    dtype=cfg.dtype, n_window=cfg.n_window)
    prm = api.Params(cfg.alpha, cfg.rho, cfg.window, cfg.base_ratio)
    assert api.kvc_plan(spec, prm)[1] > C.KVC_NOALLOC_MAX_WORKSPACE
    t = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(C.KvcError) as e:
        api.kvc_compress_noalloc(spec, prm, t, t, t, t, t, t, t, t, t)
    assert e.value.status == C.KVC_ERR_WORKSPACE
