"""The byte and flop model bench.py reports against, pinned by closed forms
(CPU only).

Per (sequence, layer, KV head) unit the path must move L d e bytes of K (the
scores), the window queries G W d e, and for the b kept rows their K and V
read and written plus a 4-byte position: 4 b d e + 4 b.  The budgets of one
pool sum exactly to N floor(retention L) (the budget invariant), so the
totals have closed forms; the score passes do 2 G W d L flops per unit and
pass.  The Omni30B-shaped workload (48 x 4 units, G W = 8 x 32, d = 128,
bf16, L = 32768, retention 0.4) gives 4 210 202 880 bytes per step.
"""
import math

import numpy as np
import pytest

import bench
from audio_kv_cache_amd import synth
from oracle import oracle as O


def _budgets(cfg, hdr):
    return np.concatenate([O.budget(hdr.head_scores, int(L), float(r), cfg.base_ratio, cfg.window)
                           for L, r in zip(hdr.lengths, hdr.retention)])


def test_omni30b_bytes_and_flops_closed_form():
    cfg = synth.CONFIGS["omni30b"]
    hdr = synth.header(cfg)
    b = _budgets(cfg, hdr)
    units, L, d, e, gw = 48 * 4, 32768, 128, 2, 8 * 32
    kbar = math.floor(0.4 * L)
    assert int(b.sum()) == units * kbar          # the budget invariant (one pool)
    m = bench.algorithmic_bytes(cfg, hdr, b)
    k_read, q_read = units * L * d * e, units * gw * d * e
    gather = 4 * units * kbar * d * e + 4 * units * kbar
    assert m["gather"] == gather
    assert m["total"] == k_read + q_read + gather == 4_210_202_880
    assert m["score_flops"] == 2 * gw * d * L * units == 412_316_860_416
    # pooling pass: K, queries, one LSE per query, the fp32 score rows
    assert m["pool"] == k_read + q_read + 4 * gw * units + 4 * L * units


@pytest.mark.parametrize("name", ["qwen7b", "long64k", "ragged"])
def test_totals_follow_the_budget_invariant(name):
    cfg = synth.CONFIGS[name]
    hdr = synth.header(cfg)
    b = _budgets(cfg, hdr)
    per_seq = cfg.n_layers * cfg.n_kv_heads
    kbars = [min(math.floor(float(r) * int(L)), int(L)) for L, r in zip(hdr.lengths, hdr.retention)]
    kept = per_seq * sum(kbars)
    assert int(b.sum()) == kept
    e = 2 if cfg.dtype == "bf16" else 4
    d, gw = cfg.head_dim, cfg.gqa * cfg.n_window
    tok = per_seq * int(sum(int(L) for L in hdr.lengths))
    m = bench.algorithmic_bytes(cfg, hdr, b)
    assert m["total"] == tok * d * e + per_seq * cfg.n_seq * gw * d * e + 4 * kept * d * e + 4 * kept
    assert m["score_flops"] == 2 * gw * d * tok


def test_decode_bytes_closed_form():
    cfg = synth.DECODE_CONFIGS["vz_omni30b"]
    m = bench.decode_bytes(cfg)
    units = cfg.n_layers * cfg.n_kv_heads * cfg.n_seq
    n, B, d, e, G = int(cfg.lens[0]), int(cfg.budgets[0]), cfg.head_dim, 2, cfg.gqa
    # logits: the cache's K, the new token's queries, A_prev
    assert m["logits"] == units * (n * d * e + G * d * e + 4 * (n - 1))
    # gather: kept K and V rows read and written, A and positions out
    assert m["gather"] == units * (4 * B * d * e + 8 * B)


_SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1399 W
        THROTTLE_STATUS: N/A
    CLOCK:
        GFX_0:
            CLK: 1723 MHz
            MIN_CLK: 500 MHz
        GFX_1:
            CLK: 1630 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_smi_sample_parses_power_and_xcd_clocks(monkeypatch):
    """The power leg's reader takes the socket power and one clock per GFX
    domain, not the memory clock or the limits."""
    class R:
        stdout, stderr, returncode = _SMI_TEXT, "", 0
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: R())
    assert bench.smi_sample() == {"socket_w": 1399.0, "gfx_mhz": [1723, 1630]}


def test_smi_sample_missing_tool(monkeypatch):
    def boom(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(bench.subprocess, "run", boom)
    assert bench.smi_sample() is None
