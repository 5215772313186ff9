"""Seeded synthetic inputs shaped like audio-LLM prefill KV caches.

This module holds input generation only -- none of the compression method's
arithmetic -- and is the single source of inputs for both the HIP path and
the CPU oracle, so both sides read identical bit patterns.

The pages measure on speech corpora (LibriSpeech, MLS, long-form recordings)
that are not available here; these generators stand in for their *shapes*:
keys and window queries carry a smooth temporal drift (audio frames are
continuous in time, AudioKV article section 1), an attention sink at the first
audio position (the WnW digest reports prefill attention concentrated on the
start of the audio), and 15-20 % of heads are audio-critical (AudioKV article
section 1.1).  No item of any corpus is reproduced.

Recipe, per (sequence, layer, KV head) unit, from its own spawned seed:
  periods P_1..P_3 ~ U[50, 400], phases phi[i, c] ~ U[0, 2 pi),
  drift[t, c] = sum_i 0.5 sin(2 pi t / P_i + phi[i, c]),
  sink direction v = normalise(N(0, I_d)),
  K[t] = N(0, I) + drift[t] + [t == 0] * beta * sqrt(d) * v,      beta = 8
  Q[g, q] = N(0, I) + drift[L + q] + v                 (g over the GQA group)
  V[t] = N(0, I)
then rounded to bf16 (round to nearest even) unless the config is fp32.
Head scores: U(0, 1) for the tiny config; otherwise round(0.18 N) randomly
chosen heads ~ U(0.6, 1) and the rest ~ U(0, 0.2).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os

import numpy as np

SINK_BETA = 8.0
DRIFT_AMP = 0.5
N_SINUSOIDS = 3
AUDIO_HEAD_FRACTION = 0.18


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int               # seeds SeedSequence(1000 + index)
    n_seq: int
    n_layers: int
    n_kv_heads: int
    gqa: int
    head_dim: int
    dtype: str               # "bf16" | "f32"
    n_window: int = 32
    alpha: float = 0.5
    rho: float = 0.7
    window: int = 32
    base_ratio: float = 0.5
    lengths: tuple = ()      # fixed per-sequence L, or () for the ragged draw
    retention: tuple = ()    # fixed per-sequence retention, or () for U(0.2,0.6)
    length_choices: tuple = ()
    sink_beta: float = SINK_BETA
    budget_pool: int = 0     # 0: one pool per sequence, 1: one pool per layer
    score_pool: int = 0      # 0: mean over the group's queries, 1: max over heads


CONFIGS = {
    "tiny": Config("tiny", 0, 1, 1, 4, 1, 64, "f32", lengths=(1024,),
                   retention=(0.6,)),
    "qwen7b": Config("qwen7b", 1, 1, 28, 4, 7, 128, "bf16", lengths=(8192,),
                     retention=(0.6,)),
    "omni30b": Config("omni30b", 2, 1, 48, 4, 8, 128, "bf16", alpha=0.6,
                      lengths=(32768,), retention=(0.4,)),
    "ragged": Config("ragged", 3, 8, 28, 4, 7, 128, "bf16",
                     length_choices=(4096, 8192, 16384, 32768)),
    "long64k": Config("long64k", 4, 1, 48, 4, 8, 128, "bf16",
                      lengths=(65536,), retention=(0.2,)),
    # an audio length that is not a power of two (40 minutes at 12.5 Hz)
    "omni30b_30000": Config("omni30b_30000", 5, 1, 48, 4, 8, 128, "bf16", alpha=0.6,
                            lengths=(30000,), retention=(0.4,)),
    # mixed lengths, none a power of two, odd and even
    "ragged_npot": Config("ragged_npot", 6, 3, 4, 2, 4, 128, "bf16",
                          lengths=(3000, 12345, 777), retention=(0.5, 0.3, 0.8)),
    # long-form audio of an odd length between 32K and 64K tokens
    "long_npot": Config("long_npot", 7, 1, 48, 4, 8, 128, "bf16",
                        lengths=(49999,), retention=(0.2,)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Header:
    """Per-config draws shared by all units: lengths, retentions, head scores."""
    cfg: Config
    lengths: np.ndarray      # int64 [n_seq]
    retention: np.ndarray    # float64 [n_seq]
    head_scores: np.ndarray  # float32 [n_layers, n_kv_heads]

    @property
    def seq_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)

    @property
    def n_units(self) -> int:
        c = self.cfg
        return c.n_seq * c.n_layers * c.n_kv_heads


def _root(cfg: Config, n_units: int):
    return np.random.SeedSequence(1000 + cfg.index).spawn(1 + n_units)


def header(cfg: Config) -> Header:
    n_units = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    rng = np.random.default_rng(_root(cfg, n_units)[0])
    if cfg.lengths:
        lengths = np.array(cfg.lengths, dtype=np.int64)
    else:
        lengths = rng.choice(np.array(cfg.length_choices, dtype=np.int64),
                             size=cfg.n_seq)
    if cfg.retention:
        retention = np.array(cfg.retention, dtype=np.float64)
    else:
        retention = rng.uniform(0.2, 0.6, size=cfg.n_seq)
    nh = cfg.n_layers * cfg.n_kv_heads
    if cfg.name == "tiny":
        S = rng.uniform(0.0, 1.0, size=nh)
    else:
        n_audio = int(round(AUDIO_HEAD_FRACTION * nh))
        audio = rng.choice(nh, size=n_audio, replace=False)
        S = rng.uniform(0.0, 0.2, size=nh)
        S[audio] = rng.uniform(0.6, 1.0, size=n_audio)
    return Header(cfg, lengths, retention,
                  S.astype(np.float32).reshape(cfg.n_layers, cfg.n_kv_heads))


def unit(cfg: Config, hdr: Header, seq: int, layer: int, head: int,
         *, sink_beta=None):
    """Generate one unit's (q [G, W, d], k [L, d], v [L, d]).

    Returns float32 arrays for fp32 configs and uint16 bf16 bit arrays
    otherwise.
    """
    beta = cfg.sink_beta if sink_beta is None else sink_beta
    u = (seq * cfg.n_layers + layer) * cfg.n_kv_heads + head
    rng = np.random.default_rng(_root(cfg, hdr.n_units)[1 + u])
    L, d, G, W = int(hdr.lengths[seq]), cfg.head_dim, cfg.gqa, cfg.n_window
    periods = rng.uniform(50.0, 400.0, size=N_SINUSOIDS)
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(N_SINUSOIDS, d))
    v = rng.standard_normal(d)
    v /= np.linalg.norm(v)
    kn = rng.standard_normal((L, d), dtype=np.float32)
    qn = rng.standard_normal((G, W, d), dtype=np.float32)
    vv = rng.standard_normal((L, d), dtype=np.float32)
    # sum_i a sin(w_i t + phi_ic) = sum_i a [sin(w_i t) cos(phi_ic) + cos(w_i t) sin(phi_ic)]
    t = np.arange(L + W, dtype=np.float64)
    w = 2.0 * math.pi / periods
    A = np.concatenate([np.sin(np.outer(t, w)), np.cos(np.outer(t, w))], axis=1)
    B = DRIFT_AMP * np.concatenate([np.cos(phases), np.sin(phases)], axis=0)
    drift = (A @ B).astype(np.float32)
    k = kn + drift[:L]
    k[0] += np.float32(beta * math.sqrt(d)) * v.astype(np.float32)
    q = qn + drift[L:L + W][None, :, :] + v.astype(np.float32)[None, None, :]
    if cfg.dtype == "f32":
        return q.astype(np.float32), k.astype(np.float32), vv
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(vv)


@dataclasses.dataclass
class Problem:
    """A whole batch in the packed layout the library takes.

    q: [n_seq, n_layers, n_kv_heads * gqa, W, d]
    k, v: [n_layers, n_kv_heads, T, d] with T = sum of lengths; sequence i
          occupies tokens seq_start[i] .. seq_start[i+1].
    """
    hdr: Header
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    @property
    def cfg(self) -> Config:
        return self.hdr.cfg


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def problem(cfg: Config, *, sink_beta=None, hdr: Header | None = None) -> Problem:
    hdr = hdr or header(cfg)
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    T = int(hdr.lengths.sum())
    NL, H, G, W, d = cfg.n_layers, cfg.n_kv_heads, cfg.gqa, cfg.n_window, cfg.head_dim
    q = np.empty((cfg.n_seq, NL, H * G, W, d), dtype=dt)
    k = np.empty((NL, H, T, d), dtype=dt)
    v = np.empty((NL, H, T, d), dtype=dt)
    starts = hdr.seq_start

    def fill(args):
        i, l, h = args
        qu, ku, vu = unit(cfg, hdr, i, l, h, sink_beta=sink_beta)
        q[i, l, h * G:(h + 1) * G] = qu
        k[l, h, starts[i]:starts[i + 1]] = ku
        v[l, h, starts[i]:starts[i + 1]] = vu

    jobs = [(i, l, h) for i in range(cfg.n_seq) for l in range(NL) for h in range(H)]
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, jobs))
    return Problem(hdr, q, k, v)


# ---------------------------------------------------------------------------
# Decode-step inputs (decayed-eviction path)
# ---------------------------------------------------------------------------
# One cache per (sequence, layer, KV head) holding n rows, the last being the
# new token.  Rows carry the same drift + first-position sink as the prefill
# keys; the new token's G query heads are N(0, I) + drift[n - 1] + v.  The
# running importance A_prev of the n - 1 older rows stands in for what
# earlier decode steps accumulated: Exp(1) * 20 / n per row (a total near
# 1 / (1 - gamma) = 20) plus U(1, 4) on the four leading rows.  Capacity
# padding rows are zero.
@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    index: int
    n_seq: int
    n_layers: int
    n_kv_heads: int
    gqa: int
    head_dim: int
    dtype: str
    lens: tuple              # rows per cache, new token included, per sequence
    budgets: tuple           # cache budget B per sequence
    capacity: int
    gamma: float = 0.95
    n_sink: int = 4
    recent_frac: float = 0.2
    sink_beta: float = SINK_BETA


DECODE_CONFIGS = {
    # parity-sized, fp32
    "vz_tiny": DecodeConfig("vz_tiny", 10, 1, 1, 4, 1, 64, "f32", lens=(300,), budgets=(200,),
                            capacity=320),
    # Omni30B-shaped steady state: a 32768-token context held at a 25 %
    # budget (8192 rows); each step appends one row and evicts one
    "vz_omni30b": DecodeConfig("vz_omni30b", 11, 1, 48, 4, 8, 128, "bf16", lens=(8193,),
                               budgets=(8192,), capacity=8200),
    # first decode step after a 40 %-retention prefill of 32768 tokens
    # (13107 rows + the new token) brought down to the 25 % budget
    "vz_first": DecodeConfig("vz_first", 12, 1, 48, 4, 8, 128, "bf16", lens=(13108,),
                             budgets=(8192,), capacity=13120),
    # mixed batch: steady state, first step after prefill, still filling,
    # exactly at budget
    "vz_ragged": DecodeConfig("vz_ragged", 13, 4, 28, 4, 7, 128, "bf16",
                              lens=(4097, 13108, 2000, 1024), budgets=(4096, 8192, 4096, 1024),
                              capacity=13120),
}


@dataclasses.dataclass
class DecodeProblem:
    """q [units, G, d]; k, v [units, capacity, d]; a_prev float32
    [units, capacity] (entries 0..n-2 meaningful)."""
    cfg: DecodeConfig
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a_prev: np.ndarray

    @property
    def n_units(self) -> int:
        c = self.cfg
        return c.n_seq * c.n_layers * c.n_kv_heads

    def seq_of(self, u: int) -> int:
        return u // (self.cfg.n_layers * self.cfg.n_kv_heads)


def decode_cache(cfg: DecodeConfig, u: int):
    """One cache's (q [G, d], k [n, d], v [n, d], a_prev [n - 1])."""
    n_units = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    rng = np.random.default_rng(np.random.SeedSequence(2000 + cfg.index).spawn(n_units)[u])
    seq = u // (cfg.n_layers * cfg.n_kv_heads)
    n, d, G = int(cfg.lens[seq]), cfg.head_dim, cfg.gqa
    periods = rng.uniform(50.0, 400.0, size=N_SINUSOIDS)
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(N_SINUSOIDS, d))
    v = rng.standard_normal(d)
    v /= np.linalg.norm(v)
    kn = rng.standard_normal((n, d), dtype=np.float32)
    qn = rng.standard_normal((G, d), dtype=np.float32)
    vv = rng.standard_normal((n, d), dtype=np.float32)
    a_prev = (rng.exponential(1.0, size=n - 1) * (20.0 / n)).astype(np.float32)
    a_prev[:min(4, n - 1)] += rng.uniform(1.0, 4.0, size=min(4, n - 1)).astype(np.float32)
    t = np.arange(n, dtype=np.float64)
    w = 2.0 * math.pi / periods
    A = np.concatenate([np.sin(np.outer(t, w)), np.cos(np.outer(t, w))], axis=1)
    B = DRIFT_AMP * np.concatenate([np.cos(phases), np.sin(phases)], axis=0)
    drift = (A @ B).astype(np.float32)
    k = kn + drift
    k[0] += np.float32(cfg.sink_beta * math.sqrt(d)) * v.astype(np.float32)
    q = qn + drift[n - 1][None, :] + v.astype(np.float32)[None, :]
    if cfg.dtype == "f32":
        return q, k, vv, a_prev
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(vv), a_prev


def decode_problem(cfg: DecodeConfig) -> DecodeProblem:
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    U = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    G, d, cap = cfg.gqa, cfg.head_dim, cfg.capacity
    q = np.zeros((U, G, d), dtype=dt)
    k = np.zeros((U, cap, d), dtype=dt)
    v = np.zeros((U, cap, d), dtype=dt)
    a = np.zeros((U, cap), dtype=np.float32)

    def fill(u):
        qu, ku, vu, au = decode_cache(cfg, u)
        n = ku.shape[0]
        q[u], k[u, :n], v[u, :n], a[u, :n - 1] = qu, ku, vu, au

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(U)))
    return DecodeProblem(cfg, q, k, v, a)


# ---------------------------------------------------------------------------
# Query-guided retrieval (C3): audio key/value caches and decode queries
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class C3Config:
    name: str
    index: int
    n_seq: int
    n_layers: int
    n_kv_heads: int
    gqa: int
    head_dim: int
    lens: tuple              # audio keys n per cache, per sequence
    budgets: tuple           # B per sequence
    capacity: int


C3_CONFIGS = {
    # parity-sized
    "c3_tiny": C3Config("c3_tiny", 20, 1, 2, 2, 4, 64, lens=(300,), budgets=(40,), capacity=320),
    # d = 128; nodes over 96 keys take the multi-workgroup path; the middle
    # sequence fits its budget (retrieval bypassed)
    "c3_mixed": C3Config("c3_mixed", 21, 3, 1, 2, 8, 128, lens=(1000, 37, 2500),
                         budgets=(100, 64, 200), capacity=2560),
    # empty cache, a root that cannot split, the smallest splittable root,
    # a 97-key root (the smallest multi-workgroup node), a budget of 1
    "c3_edge": C3Config("c3_edge", 22, 5, 1, 1, 2, 64, lens=(0, 4, 5, 97, 150),
                        budgets=(1, 1, 2, 10, 1), capacity=160),
    # Qwen3-Omni-30B-A3B shape (48 layers, 4 KV heads, 8 query heads per KV
    # head, head_dim 128) at a 32K-token audio context and a 512-key budget
    "c3_omni30b": C3Config("c3_omni30b", 23, 1, 48, 4, 8, 128, lens=(32768,), budgets=(512,),
                           capacity=32768),
}


def c3_cache(cfg: C3Config, u: int):
    """One cache's audio keys and values (bf16 bits [n, d]): noise plus a slow
    drift along the audio (as for the prefill inputs) and a sink on row 0."""
    n_units = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    rng = np.random.default_rng(np.random.SeedSequence(3000 + cfg.index).spawn(n_units)[u])
    seq = u // (cfg.n_layers * cfg.n_kv_heads)
    n, d = int(cfg.lens[seq]), cfg.head_dim
    periods = rng.uniform(50.0, 400.0, size=N_SINUSOIDS)
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(N_SINUSOIDS, d))
    sink = rng.standard_normal(d)
    sink /= np.linalg.norm(sink)
    kn = rng.standard_normal((n, d), dtype=np.float32)
    vv = rng.standard_normal((n, d), dtype=np.float32)
    t = np.arange(n, dtype=np.float64)
    w = 2.0 * math.pi / periods
    A = np.concatenate([np.sin(np.outer(t, w)), np.cos(np.outer(t, w))], axis=1)
    B = DRIFT_AMP * np.concatenate([np.cos(phases), np.sin(phases)], axis=0)
    k = kn + (A @ B).astype(np.float32)
    if n:
        k[0] += np.float32(SINK_BETA * math.sqrt(d)) * sink.astype(np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(vv)


def c3_problem(cfg: C3Config):
    """k, v bf16 bits [units, capacity, d] (rows past n are zero)."""
    U = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    k = np.zeros((U, cfg.capacity, cfg.head_dim), dtype=np.uint16)
    v = np.zeros((U, cfg.capacity, cfg.head_dim), dtype=np.uint16)

    def fill(u):
        ku, vu = c3_cache(cfg, u)
        k[u, :ku.shape[0]], v[u, :vu.shape[0]] = ku, vu

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(U)))
    return k, v


def c3_queries(cfg: C3Config, step: int) -> np.ndarray:
    """Decode-step queries, bf16 bits [units, G, d]."""
    U = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    rng = np.random.default_rng(np.random.SeedSequence([4000 + cfg.index, step]))
    return f32_to_bf16_bits(rng.standard_normal((U, cfg.gqa, cfg.head_dim), dtype=np.float32))


# ---------------------------------------------------------------------------
# Decode-time chunk recall (WnW): audio caches, head roles, anchor queries
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class WnwConfig:
    name: str
    index: int
    n_seq: int
    n_layers: int
    n_kv_heads: int
    gqa: int
    head_dim: int
    lens: tuple              # audio tokens n per sequence
    capacity: int
    anchors: tuple           # units l * n_kv_heads + h with the anchor role
    fixed: tuple = ()        # units with the fixed role; every other unit is tidal


WNW_FOCUS = 2.0     # query gain on the attended keys' mean (see wnw_queries)
WNW_SPAN = 4        # attended keys per anchor query
WNW_DRIFT = 4       # positions the attended span moves per step (about 0.3 s)
WNW_JUMP = 16       # every WNW_JUMP steps the span jumps to a new place

WNW_CONFIGS = {
    # parity-sized: a short last block (317 = 12 * 25 + 17)
    "wnw_tiny": WnwConfig("wnw_tiny", 30, 1, 2, 2, 2, 64, lens=(317,), capacity=320,
                          anchors=(0,), fixed=(2,)),
    # d = 128, three sequences (one of a single chunk), two anchors
    "wnw_mixed": WnwConfig("wnw_mixed", 31, 3, 3, 2, 4, 128, lens=(1000, 51, 2503),
                           capacity=2560, anchors=(0, 3), fixed=(5,)),
    # one token, under one block, exactly one chunk, a chunk and a half
    "wnw_edge": WnwConfig("wnw_edge", 32, 4, 1, 3, 1, 64, lens=(1, 24, 50, 76), capacity=80,
                          anchors=(1,)),
    # Voxtral-Mini-3B shape (30 layers, 8 KV heads, 4 query heads per KV
    # head, head_dim 128): 5 anchor heads in the middle layers and 235 tidal
    # heads, at a 32K-token audio context (about 44 minutes at 12.5 tokens/s)
    "wnw_voxtral3b": WnwConfig("wnw_voxtral3b", 33, 1, 30, 8, 4, 128, lens=(32768,),
                               capacity=32768, anchors=(100, 109, 118, 127, 136)),
    # more than 16 query heads per KV head: a partial second block of 16
    # heads (d = 64), and two full blocks (d = 128, two sequences)
    "wnw_g20": WnwConfig("wnw_g20", 34, 1, 2, 2, 20, 64, lens=(613,), capacity=640,
                         anchors=(0, 3)),
    "wnw_g32": WnwConfig("wnw_g32", 35, 2, 1, 3, 32, 128, lens=(400, 1207), capacity=1216,
                         anchors=(1,)),
}


def wnw_roles(cfg: WnwConfig) -> np.ndarray:
    r = np.full(cfg.n_layers * cfg.n_kv_heads, 2, np.uint8)
    r[list(cfg.fixed)] = 0
    r[list(cfg.anchors)] = 1
    return r


def wnw_cache(cfg: WnwConfig, u: int):
    """One unit's audio keys and values (bf16 bits [n, d]): noise plus a slow
    drift along the audio and a sink on row 0, as for C3."""
    n_units = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    rng = np.random.default_rng(np.random.SeedSequence(5000 + cfg.index).spawn(n_units)[u])
    seq = u // (cfg.n_layers * cfg.n_kv_heads)
    n, d = int(cfg.lens[seq]), cfg.head_dim
    periods = rng.uniform(50.0, 400.0, size=N_SINUSOIDS)
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(N_SINUSOIDS, d))
    sink = rng.standard_normal(d)
    sink /= np.linalg.norm(sink)
    kn = rng.standard_normal((n, d), dtype=np.float32)
    vv = rng.standard_normal((n, d), dtype=np.float32)
    t = np.arange(n, dtype=np.float64)
    w = 2.0 * math.pi / periods
    A = np.concatenate([np.sin(np.outer(t, w)), np.cos(np.outer(t, w))], axis=1)
    B = DRIFT_AMP * np.concatenate([np.cos(phases), np.sin(phases)], axis=0)
    k = kn + (A @ B).astype(np.float32)
    k[0] += np.float32(SINK_BETA * math.sqrt(d)) * sink.astype(np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(vv)


def wnw_anchor_keys(cfg: WnwConfig) -> np.ndarray:
    """Anchor units' keys, bf16 bits [n_seq, n_anchor, capacity, d] (rows past n zero)."""
    upseq = cfg.n_layers * cfg.n_kv_heads
    out = np.zeros((cfg.n_seq, len(cfg.anchors), cfg.capacity, cfg.head_dim), np.uint16)
    for i in range(cfg.n_seq):
        for a, un in enumerate(sorted(cfg.anchors)):
            k, _ = wnw_cache(cfg, i * upseq + un)
            out[i, a, :k.shape[0]] = k
    return out


def wnw_queries(cfg: WnwConfig, step: int, k_anchor_bits: np.ndarray) -> np.ndarray:
    """Anchor queries of one decode step, bf16 bits [n_seq, n_anchor, G, d]:
    FOCUS times the mean of WNW_SPAN consecutive keys of the anchor (a span
    that moves WNW_DRIFT positions per step and jumps every WNW_JUMP steps)
    plus unit noise, so each anchor attends mostly to one moving stretch."""
    nA, G, d = len(cfg.anchors), cfg.gqa, cfg.head_dim
    out = np.zeros((cfg.n_seq, nA, G, d), np.float32)
    for i in range(cfg.n_seq):
        n = int(cfg.lens[i])
        hop = np.random.default_rng(np.random.SeedSequence([5200 + cfg.index, i, step // WNW_JUMP]))
        start = int(hop.integers(0, n))
        c = (start + WNW_DRIFT * (step % WNW_JUMP)) % n
        rng = np.random.default_rng(np.random.SeedSequence([5100 + cfg.index, i, step]))
        for a in range(nA):
            k = bf16_bits_to_f32(k_anchor_bits[i, a, :n])
            lo = min(c, max(0, n - WNW_SPAN))
            mu = k[lo:lo + WNW_SPAN].mean(axis=0)
            out[i, a] = WNW_FOCUS * mu[None, :] + rng.standard_normal((G, d), dtype=np.float32)
    return f32_to_bf16_bits(out)


def wnw_host_copies(cfg: WnwConfig, fast: bool = False):
    """K and V of every unit, bf16 bits [units, capacity, d] (the tidal heads'
    host copies are read from it).  fast: uniform random bits in place of
    the cache model (for timing, where only the bytes matter)."""
    U = cfg.n_seq * cfg.n_layers * cfg.n_kv_heads
    shape = (U, cfg.capacity, cfg.head_dim)
    if fast:
        rng = np.random.default_rng(np.random.SeedSequence(5300 + cfg.index))
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16), \
            rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    k = np.zeros(shape, np.uint16)
    v = np.zeros(shape, np.uint16)

    def fill(u):
        ku, vu = wnw_cache(cfg, u)
        k[u, :ku.shape[0]], v[u, :vu.shape[0]] = ku, vu

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(U)))
    return k, v
