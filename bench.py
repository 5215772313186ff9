"""Throughput of audio prefill KV-cache compression on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config omni30b]

One step = one kvc_compress call over the whole batch (all layers, KV heads
and sequences): scores -> spectral smoothing -> budget -> top-k -> gather,
inputs resident in HBM.  Prints one JSON line on stdout; progress on stderr.

Metric: compressed tokens*heads per second (sum of L * layers * KV heads per
step time) and the fraction of HBM peak that the path's algorithmic bytes
reach.  Algorithmic bytes per (sequence, layer, KV head) unit:
    L d e            K read once for the scores
  + 2 b d e          kept K and V rows read
  + 2 b d e          kept K and V rows written
  + 4 b              kept positions written
  + G W d e          window queries read
(e = element size, b = the unit's budget); V is never read for the scores and
the score rows are workspace.

The same line carries three decode-time legs under "decode", "retrieval"
and "recall" (decayed eviction, query-guided retrieval, chunk recall), each
timed on its own workload; --no-decode, --no-c3 and --no-wnw skip them.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import pathlib
import re
import subprocess
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
# MI355X dense matrix peaks, TFLOP/s: bf16 MFMA; fp32 inputs run on the fp64
# MFMA (78.6 TFLOP/s dense fp64)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 78.6}
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one wave64
# instruction per SIMD per 4 cycles (T lane-ops/s).
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
ROOT = pathlib.Path(__file__).resolve().parent


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, hdr, budgets):
    e = 2 if cfg.dtype == "bf16" else 4
    d = cfg.head_dim
    gw = cfg.gqa * cfg.n_window
    per_seq_units = cfg.n_layers * cfg.n_kv_heads
    n_units = per_seq_units * cfg.n_seq
    tok = sum(int(L) for L in hdr.lengths) * per_seq_units      # sum of L over units
    k_read = tok * d * e
    q_read = gw * d * e * n_units
    b = np.asarray(budgets, dtype=np.int64)
    kept = int(b.sum())
    gather = 4 * kept * d * e + 4 * kept
    return dict(
        total=k_read + gather + q_read, gather=gather,
        # pooling pass: K and the window queries read, one LSE per query read,
        # the fp32 score rows written
        pool=k_read + q_read + 4 * gw * n_units + 4 * tok,
        # statistics pass: K and queries read, one (max, sum) pair per query
        # and score tile (SCORE_TILE_KEYS keys) written
        stats=k_read + q_read + 8 * gw * sum(-(-int(L) // SCORE_TILE_KEYS) for L in hdr.lengths)
        * per_seq_units,
        # both passes: one G*W x d by d x L product per unit
        score_flops=2 * gw * d * tok)


# keys per score workgroup in the library (KVC_TILE_KEYS)
SCORE_TILE_KEYS = 2048


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        h.update((ROOT / "audio_kv_cache_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


def committed_traffic(kernel_file: str, kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it matches the
    current kernel source; None otherwise."""
    p = ROOT / "profiles" / "traffic.json"
    if not p.exists():
        return None
    try:
        rec = json.loads(p.read_text()).get(f"{workload}:{kernel}")
    except json.JSONDecodeError:
        return None
    if not rec or rec.get("source_sha") != source_hash(kernel_file):
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, hdr, prob_units, budgets, max_units=16):
    """The fp64 oracle, as it stands, on a bounded sample of units: the
    first max_units units of sequence 0 (layer 0's KV heads, then layer 1's)
    on a thread pool of min(max_units, usable cores) threads, and the first
    unit alone on one thread.  BLAS inside the oracle is held to one thread
    so the pool size is the number of cores used."""
    from oracle import oracle as O
    from audio_kv_cache_amd import synth
    import concurrent.futures as cf
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    affinity = O.threads()
    units = [x for x in prob_units if x[0] == 0][:max_units]
    cores = min(len(units), affinity)
    # regenerate only the sampled units (each is seeded on its own)
    inputs = [synth.unit(cfg, hdr, i, l, h) for (i, l, h) in units]

    def run(j):
        (i, l, h), (qu, ku, _) = units[j], inputs[j]
        u = (i * cfg.n_layers + l) * cfg.n_kv_heads + h
        O.unit_compress(qu, ku, cfg.dtype, int(budgets[u]), cfg.alpha, cfg.rho, cfg.window)

    limit = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        t0 = time.perf_counter()
        run(0)
        dt1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(cores) as ex:
            list(ex.map(run, range(len(units))))
        dt = time.perf_counter() - t0
    finally:
        if limit is not None:
            limit.unregister()
    L0 = int(hdr.lengths[0])
    toks = L0 * len(units)
    layers = sorted({l for (_, l, _) in units})
    return dict(value=toks / dt, unit="tokens·heads/s", cores=cores, kind="oracle",
                sample=f"subset: {len(units)} units (sequence 0, layers {layers[0]}-{layers[-1]}, "
                       f"all KV heads) of the same workload, scores+smoothing+selection in fp64, "
                       f"{dt:.1f} s wall on {cores} threads; one unit on one thread {dt1:.1f} s",
                one_thread_value=L0 / dt1, affinity_cores=affinity, cpu_model=cpu_model())


def summed_traffic(kernel_file: str, kernels, workload: str):
    """Sum of committed_traffic over a step's kernels (None if any is missing)."""
    parts = [committed_traffic(kernel_file, k, workload) for k in kernels]
    return None if any(x is None for x in parts) else sum(parts)


def decode_bytes(cfg):
    """Algorithmic bytes of one decode step: per cache, K read once for the
    logits, the new token's queries, A_prev read, kept K and V rows read and
    written, A_out and the kept positions written."""
    e = 2 if cfg.dtype == "bf16" else 4
    d, G = cfg.head_dim, cfg.gqa
    per_seq = cfg.n_layers * cfg.n_kv_heads
    tot = dict(logits=0, gather=0, total=0)
    for n, B in zip(cfg.lens, cfg.budgets):
        nl = min(n, B)
        lg = n * d * e + G * d * e + 4 * (n - 1)
        ga = 4 * nl * d * e + 8 * nl
        tot["logits"] += per_seq * lg
        tot["gather"] += per_seq * ga
        tot["total"] += per_seq * (lg + ga)
    return tot


def bench_decode(args):
    """One decode step of decayed eviction (kvc_vz_step) over every cache of
    the decode workload, inputs resident in HBM; per-kernel event timing and
    a CPU-oracle sample."""
    gc.collect()
    import torch
    from audio_kv_cache_amd import api, synth
    cfg = synth.DECODE_CONFIGS[args.decode_config]
    log(f"[bench] decode: generating {cfg.name}")
    prob = synth.decode_problem(cfg)

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v = dev(prob.q), dev(prob.k), dev(prob.v)
    a_prev = torch.from_numpy(prob.a_prev).cuda()
    spec = api.VzSpec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                      head_dim=cfg.head_dim, lens=cfg.lens, budgets=cfg.budgets,
                      capacity=cfg.capacity, dtype=cfg.dtype)
    prm = api.VzParams(cfg.gamma, cfg.n_sink, cfg.recent_frac)
    _, wsb = api.kvc_vz_plan(spec, prm)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ko, vo = torch.empty_like(k), torch.empty_like(v)
    ao = torch.empty_like(a_prev)
    at = torch.empty_like(a_prev)
    idx = torch.empty(a_prev.shape, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps

    step_ms = timed(lambda: api.kvc_vz_step(spec, prm, q, k, v, a_prev, ko, vo, ao, idx, ws,
                                            stream))
    stages = {
        "accumulate": timed(lambda: api.kvc_vz_accumulate(spec, prm, q, k, a_prev, at, ws,
                                                          stream)),
        "evict": timed(lambda: api.kvc_vz_evict(spec, prm, at, idx, stream)),
        "gather": timed(lambda: api.kvc_vz_gather(spec, prm, k, v, at, idx, ko, vo, ao,
                                                  stream)),
    }
    # The same step with the caches kept in place (kvc_vz_step_inplace),
    # where every cache gives up at most one row: a holds A_prev with the new
    # token's slot at 0, pos the compact order.  Each timed call decays A,
    # frees one slot and gives it the next place, so consecutive calls do
    # the same work.
    inplace = None
    if all(int(n) <= int(b) + 1 for n, b in zip(cfg.lens, cfg.budgets)):
        a_np = prob.a_prev.copy()
        pos_np = np.full(a_np.shape, -1, dtype=np.int32)
        for u in range(prob.n_units):
            n = int(cfg.lens[prob.seq_of(u)])
            a_np[u, n - 1] = 0.0
            pos_np[u, :n] = np.arange(n)
        a_in = torch.from_numpy(a_np).cuda()
        pos_in = torch.from_numpy(pos_np).cuda()
        free = torch.empty(prob.n_units, dtype=torch.int32, device="cuda")
        in_ms = timed(lambda: api.kvc_vz_step_inplace(spec, prm, q, k, a_in, pos_in, free, ws,
                                                      stream))
        in_scrub_ms = scrubbed_ms(lambda i: api.kvc_vz_step_inplace(spec, prm, q, k, a_in, pos_in,
                                                                    free, ws, stream),
                                  args.steps, stream)
        ib = 0
        for n in cfg.lens:
            ib += cfg.n_layers * cfg.n_kv_heads * (n * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
                                                   + cfg.gqa * cfg.head_dim * 2 + 12 * n + 4)
        i_gbs = ib / (in_ms * 1e-3) / 1e9
        inplace = {"us_per_step": round(in_ms * 1e3, 2),
                   "us_per_step_scrubbed": round(in_scrub_ms * 1e3, 2),
                   "traffic": summed_traffic("voxzip.hip", ("vz_logits_bf16_kernel", "vz_accum_kernel",
                                                            "vz_slot_evict_kernel"), cfg.name),
                   "cache_rows_per_s": sum(int(n) for n in cfg.lens) * cfg.n_layers
                   * cfg.n_kv_heads / (in_ms * 1e-3),
                   "algorithmic_bytes_per_step": ib,
                   "path_hbm": {"achieved": round(i_gbs, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(i_gbs / HBM_PEAK_GBS, 4)}}
        log(f"[bench] decode in place {in_ms * 1e3:.1f} us/step, path {i_gbs:.0f} GB/s; "
            f"{in_scrub_ms * 1e3:.1f} us after a cache scrub")
    step_scrub_ms = scrubbed_ms(lambda i: api.kvc_vz_step(spec, prm, q, k, v, a_prev, ko, vo, ao,
                                                          idx, ws, stream), args.steps, stream)
    ab = decode_bytes(cfg)
    units = prob.n_units
    rows = sum(int(n) for n in cfg.lens) * cfg.n_layers * cfg.n_kv_heads
    gbs = ab["total"] / (step_ms * 1e-3) / 1e9
    g_gbs = ab["gather"] / (stages["gather"] * 1e-3) / 1e9
    a_gbs = ab["logits"] / (stages["accumulate"] * 1e-3) / 1e9
    log(f"[bench] decode {step_ms * 1e3:.1f} us/step ({step_scrub_ms * 1e3:.1f} us after a cache "
        f"scrub), path {gbs:.0f} GB/s; stages " +
        ", ".join(f"{n2} {t * 1e3:.1f} us" for n2, t in stages.items()))
    out = {
        "workload": f"{cfg.name}: {units} caches ({cfg.n_seq} seq x {cfg.n_layers} layers x "
                    f"{cfg.n_kv_heads} KV heads), n={list(cfg.lens)} rows, budget "
                    f"{list(cfg.budgets)}, GQA {cfg.gqa}, head_dim {cfg.head_dim}, {cfg.dtype}, "
                    f"gamma {cfg.gamma}, T {cfg.n_sink}, recent {cfg.recent_frac}",
        "us_per_step": round(step_ms * 1e3, 2),
        "us_per_step_scrubbed": round(step_scrub_ms * 1e3, 2),
        "cache_rows_per_s": rows / (step_ms * 1e-3),
        "algorithmic_bytes_per_step": ab["total"],
        "path_hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "stage_us": {n2: round(t * 1e3, 2) for n2, t in stages.items()},
        "roofline": {"gather": {"bound": "hbm", "kernel": "vz_gather_kernel<256>",
                                "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                                "traffic": committed_traffic("voxzip.hip", "vz_gather_kernel",
                                                             cfg.name)},
                     "accumulate": {"bound": "hbm",
                                    "kernel": "vz_logits_bf16_kernel + vz_accum_kernel",
                                    "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4)}},
        "inplace": inplace,
    }
    if not args.no_cpu_baseline:
        from oracle import voxzip as VZ
        from oracle import oracle as O
        import concurrent.futures as cf
        sample = list(range(min(64, units)))
        cores = min(len(sample), O.threads())

        def run(u):
            n = int(cfg.lens[prob.seq_of(u)])
            B = int(cfg.budgets[prob.seq_of(u)])
            VZ.step(O.widen(prob.q[u], cfg.dtype), O.widen(prob.k[u, :n], cfg.dtype),
                    prob.v[u, :n], prob.a_prev[u, :n - 1].astype(np.float64), B, cfg.gamma,
                    cfg.n_sink, cfg.recent_frac)

        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(cores) as ex:
            list(ex.map(run, sample))
        dt = time.perf_counter() - t0
        srows = sum(int(cfg.lens[prob.seq_of(u)]) for u in sample)
        out["cpu_baseline"] = dict(value=srows / dt, unit="cache rows/s", cores=cores,
                                   kind="oracle",
                                   sample=f"{len(sample)} caches of the same workload, one "
                                          f"decode step each in fp64, {dt:.2f} s wall")
    del prob
    return out


def c3_bytes(cfg, A_total, kept_total):
    """Algorithmic HBM bytes of one C3 decode step: every frontier entry's
    centroid (bf16), id and score once; every kept K and V row read and
    written once, with its position."""
    d = cfg.head_dim
    score = A_total * (2 * d + 4 + 4)
    select = A_total * (4 + 4 + 8 + 4) + kept_total * 4
    gather = kept_total * (2 * 2 * 2 * d + 4)
    return {"score": score, "select_update": select, "gather": gather,
            "total": score + select + gather}


def bench_c3(args):
    """C3 retrieval: the prefill tree build over every cache and the decode
    step (scores, budget fill, frontier update, gather), inputs resident in
    HBM; per-kernel event timing and a CPU-oracle sample."""
    gc.collect()
    import torch
    from audio_kv_cache_amd import api, synth
    cfg = synth.C3_CONFIGS[args.c3_config]
    log(f"[bench] c3: generating {cfg.name}")
    k_np, v_np = synth.c3_problem(cfg)
    k = torch.from_numpy(k_np.view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(v_np.view(np.int16)).cuda().view(torch.bfloat16)
    spec = api.C3Spec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                      head_dim=cfg.head_dim, lens=cfg.lens, budgets=cfg.budgets,
                      capacity=cfg.capacity)
    prm = api.C3Params()
    o = api.c3_allocate(spec, prm, "cuda")
    stream = torch.cuda.current_stream()
    U = spec.n_units
    log("[bench] c3: building")
    api.kvc_c3_build(spec, prm, k, o["index"], o["state"][0], o["build_ws"], stream)
    builds = []
    for _ in range(max(1, args.c3_builds)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        api.kvc_c3_build(spec, prm, k, o["index"], o["state"][0], o["build_ws"], stream)
        torch.cuda.synchronize()
        builds.append(time.perf_counter() - t0)
    build_ms = 1e3 * sorted(builds)[len(builds) // 2]
    V = api.C3Views(spec, o["layout"], o["index"], o["state"][0])
    left = V.left.cpu().numpy()
    size = V.size.cpu().numpy()
    nn = V.n_nodes.cpu().numpy()
    split_keys = sum(int(size[u, :nn[u]][left[u, :nn[u]] >= 0].sum()) for u in range(U))
    A_total = int(V.count.sum().item())
    kept_total = sum(min(int(cfg.lens[u // (cfg.n_layers * cfg.n_kv_heads)]),
                         int(cfg.budgets[u // (cfg.n_layers * cfg.n_kv_heads)])) for u in range(U))
    keys = sum(int(n) for n in cfg.lens) * cfg.n_layers * cfg.n_kv_heads
    # Build: 8 Lloyd iterations over the keys of every node that splits; per
    # key and iteration d multiply-adds for the hyperplane test and d adds
    # for the member sums.
    build_ops = split_keys * 8 * 2 * cfg.head_dim
    build_tops = build_ops / (build_ms * 1e-3) / 1e12
    log(f"[bench] c3 build {build_ms:.2f} ms ({keys / (build_ms * 1e-3):.4g} keys/s, "
        f"{build_tops:.2f} T lane-ops/s), {int(nn.sum())} nodes, frontier {A_total}")

    qs = [torch.from_numpy(synth.c3_queries(cfg, s).view(np.int16)).cuda().view(torch.bfloat16)
          for s in range(4)]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = [0]

    def step(i, st=stream):
        si, so = o["state"][cur[0]], o["state"][1 - cur[0]]
        api.kvc_c3_step(spec, prm, o["index"], si, so, qs[i % 4], k, v, o["k_out"], o["v_out"],
                        o["idx"], o["step_ws"], st)
        cur[0] = 1 - cur[0]

    def timed(fn, n):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(n):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    step_ms = timed(step, args.steps)
    # the same steps replayed from one captured graph
    graph_step_ms = graph_ms(lambda: [step(i, None) for i in range(args.steps)], args.steps)
    scrub_step_ms = scrubbed_ms(step, args.steps, stream)
    si = o["state"][cur[0]]
    so = o["state"][1 - cur[0]]
    stages = {
        "score": timed(lambda i: api.kvc_c3_score(spec, prm, o["index"], si, qs[0], o["sigma"],
                                                  stream), args.steps),
        "select": timed(lambda i: api.kvc_c3_select(spec, prm, o["index"], si, o["sigma"],
                                                    o["idx"], stream), args.steps),
        "update": timed(lambda i: api.kvc_c3_update(spec, prm, o["index"], si, o["sigma"], so,
                                                    stream), args.steps),
        "gather": timed(lambda i: api.kvc_c3_gather(spec, prm, k, v, o["idx"], o["k_out"],
                                                    o["v_out"], stream), args.steps),
    }
    ab = c3_bytes(cfg, A_total, kept_total)
    gbs = {n2: ab[n3] / (stages[n2] * 1e-3) / 1e9 for n2, n3 in
           (("score", "score"), ("gather", "gather"))}
    log(f"[bench] c3 step {step_ms * 1e3:.1f} us ({graph_step_ms * 1e3:.1f} us from a graph, "
        f"{scrub_step_ms * 1e3:.1f} us after a cache scrub); stages " +
        ", ".join(f"{n2} {t * 1e3:.1f} us" for n2, t in stages.items()))

    def hbm(kernel, g, src):
        return {"bound": "hbm", "kernel": kernel, "achieved": round(g, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(g / HBM_PEAK_GBS, 4),
                "traffic": committed_traffic(src, kernel.split("<")[0], cfg.name)}

    out = {
        "workload": f"{cfg.name}: {U} caches ({cfg.n_seq} seq x {cfg.n_layers} layers x "
                    f"{cfg.n_kv_heads} KV heads), n={list(cfg.lens)} audio keys, budget "
                    f"{list(cfg.budgets)}, GQA {cfg.gqa}, head_dim {cfg.head_dim}, bf16, "
                    f"lambda {prm.lam}, R {prm.r_swaps}",
        "build_ms": round(build_ms, 3),
        "build_keys_per_s": keys / (build_ms * 1e-3),
        "build_roofline": {"bound": "alu", "kernels": "c3_local_kernel + c3_span_* (whole build)",
                           "achieved": round(build_tops, 3), "peak": VALU_PEAK_TOPS,
                           "unit": "T lane-ops/s", "frac": round(build_tops / VALU_PEAK_TOPS, 4),
                           "ops": build_ops},
        "nodes": int(nn.sum()), "frontier_entries": A_total,
        "us_per_step": round(step_ms * 1e3, 2),
        "us_per_step_graph": round(graph_step_ms * 1e3, 2),
        "us_per_step_scrubbed": round(scrub_step_ms * 1e3, 2),
        "steps_per_s": 1e3 / step_ms,
        "algorithmic_bytes_per_step": ab["total"],
        "stage_us": {n2: round(t * 1e3, 2) for n2, t in stages.items()},
        "roofline": {"score": hbm(f"c3_score_kernel<{cfg.head_dim}, 8>", gbs["score"], "c3.hip"),
                     "gather": hbm(f"c3_gather_kernel<{cfg.head_dim}>", gbs["gather"], "c3.hip")},
    }
    if not args.no_cpu_baseline:
        from oracle import c3 as C3
        u = 0
        n = int(cfg.lens[0])
        Kf = synth.bf16_bits_to_f32(k_np[u, :n]).astype(np.float64)
        t0 = time.perf_counter()
        tree = C3.build_tree(Kf, cache=u)
        tb = time.perf_counter() - t0
        F = C3.initial_frontier(tree, n)
        e = np.zeros(len(F))
        q0 = synth.bf16_bits_to_f32(synth.c3_queries(cfg, 0)[u]).astype(np.float64)
        t0 = time.perf_counter()
        nst = 5
        for _ in range(nst):
            r = C3.step(tree, F, e, q0, n, int(cfg.budgets[0]))
            F, e = r["F"], r["e"]
        ts = (time.perf_counter() - t0) / nst
        out["cpu_baseline"] = dict(value=n / tb,
                                   unit="keys/s (tree build)", cores=1, kind="oracle",
                                   sample=f"cache 0 of the same workload: tree build of {n} keys "
                                          f"{tb:.2f} s; one decode step {ts * 1e3:.2f} ms "
                                          f"(about {U * ts:.2f} s for all {U} caches)",
                                   step_caches_per_s=1.0 / ts)
    del k_np, v_np
    return out


PCIE_PEAK_GBS = 64.0        # PCIe 5.0 x16, one direction (the MI355X host link)


def smi_sample():
    """Socket power (W) and per-XCD shader clocks (MHz) as amd-smi reads them now,
    or None where the tool is missing or prints neither."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                           timeout=30)
    except (OSError, subprocess.TimeoutExpired):
        return None
    power = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", r.stdout)
    clocks = [int(c) for c in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", r.stdout)]
    if power is None and not clocks:
        return None
    return {"socket_w": float(power.group(1)) if power else None, "gfx_mhz": clocks}


def power_sample(calls, ms_each, seconds, sync):
    """Keep each call looping on the GPU for about `seconds` and read socket power
    and shader clocks halfway through: which stages run at the power cap and
    at what clock.  Diagnostic only; nothing here is timed."""
    res = {}
    for name, fn in calls.items():
        n = max(1, int(seconds * 1e3 / max(ms_each[name], 1e-3)))
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        time.sleep(max(0.0, seconds / 2 - (time.perf_counter() - t0)))
        res[name] = smi_sample()
        sync()
        if res[name] is None:
            log("[bench] power: amd-smi gave no reading")
            return res
        c = res[name]["gfx_mhz"]
        log(f"[bench] power {name}: socket {res[name]['socket_w']} W, shader clocks "
            f"{min(c) if c else '-'}-{max(c) if c else '-'} MHz over {len(c)} XCDs")
        time.sleep(0.5)
    return res


def graph_ms(issue, n):
    """Capture issue() (n steps launched on the current stream) into one HIP
    graph, replay it once, and return the event time per step."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        issue()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n


_SCRUB = []


def scrubbed_ms(fn, n, stream):
    """Mean event time of n calls fn(i), each after a 512 MiB device-to-device
    copy (1 GiB of traffic) that evicts the 256 MB memory-side cache, as the
    other work of a serving step between two decode steps would."""
    import torch
    if not _SCRUB:
        _SCRUB.extend(torch.empty(512 << 20, dtype=torch.uint8, device="cuda") for _ in range(2))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i in range(n):
        _SCRUB[1].copy_(_SCRUB[0])
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / n


def bench_wnw(args):
    """WnW chunk recall: one decode step (anchor chunk scores, top-3 with
    release hysteresis, slot update, recall of newly resident blocks of every
    tidal head from page-locked host memory), inputs resident (anchor keys
    in HBM, tidal copies in host memory); per-stage event timing, the bytes
    recalled per step, a cold step (everything recalled), CPU-oracle sample."""
    gc.collect()
    import torch
    from audio_kv_cache_amd import api, synth
    cfg = synth.WNW_CONFIGS[args.wnw_config]
    prm = api.WnwParams()
    S = prm.chunk_stride
    log(f"[bench] wnw: generating {cfg.name}")
    roles = synth.wnw_roles(cfg)
    spec = api.WnwSpec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                       head_dim=cfg.head_dim, lens=cfg.lens, roles=roles, capacity=cfg.capacity,
                       slot_rows=prm.slot_cap * S)
    ka = synth.wnw_anchor_keys(cfg)
    U, upseq, d = spec.n_units, cfg.n_layers * cfg.n_kv_heads, cfg.head_dim
    k = torch.zeros((U, cfg.capacity, d), dtype=torch.int16, device="cuda")
    for i in range(cfg.n_seq):
        for a, un in enumerate(sorted(cfg.anchors)):
            k[i * upseq + un] = torch.from_numpy(ka[i, a].view(np.int16)).cuda()
    kh_np, vh_np = synth.wnw_host_copies(cfg, fast=True)
    hk = torch.empty(kh_np.shape, dtype=torch.int16, pin_memory=True)
    hv = torch.empty(vh_np.shape, dtype=torch.int16, pin_memory=True)
    hk.copy_(torch.from_numpy(kh_np.view(np.int16)))
    hv.copy_(torch.from_numpy(vh_np.view(np.int16)))
    del kh_np, vh_np
    o = api.wnw_allocate(spec, prm, "cuda")
    lay = o["layout"]
    stream = torch.cuda.current_stream()
    n_steps = args.warmup + args.steps
    qs = [torch.from_numpy(synth.wnw_queries(cfg, t, ka).view(np.int16)).cuda()
          for t in range(n_steps)]
    cur = [0]

    def reset():
        for st in o["state"]:
            api.kvc_wnw_init(spec, prm, st, stream)
        cur[0] = 0

    def step(t, st=stream):
        si, so = o["state"][cur[0]], o["state"][1 - cur[0]]
        api.kvc_wnw_step(spec, prm, qs[t], k, si, so, hk, hv, o["slot_k"], o["slot_v"],
                         o["sigma"], o["ws"], st)
        cur[0] = 1 - cur[0]

    # Pass 1, untimed: the blocks recalled by each step.
    reset()
    rec_blocks = []
    for t in range(n_steps):
        step(t)
        torch.cuda.synchronize()
        V = api.WnwViews(spec, prm, lay, o["state"][cur[0]])
        nrec = V.n_recalled.cpu().numpy()
        rb = V.recalled_block.cpu().numpy()
        rows = 0
        for i, n in enumerate(cfg.lens):
            for r in range(int(nrec[i])):
                rows += min(S, int(n) - int(rb[i, r]) * S)
        rec_blocks.append((int(nrec.sum()), rows))
    row_bytes = 2 * d * 2 * int(lay.n_tidal)          # K and V rows of every tidal head
    timed_rows = sum(r for _, r in rec_blocks[args.warmup:])
    bytes_per_step = timed_rows * row_bytes / args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Pass 2, timed: the same steps from the same state.
    reset()
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    ev0.record(stream)
    for t in range(args.warmup, n_steps):
        step(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    step_ms = ev0.elapsed_time(ev1) / args.steps
    # Pass 3: the same timed steps from the same state, replayed from one graph.
    reset()
    for t in range(args.warmup):
        step(t)
    graph_step_ms = graph_ms(lambda: [step(t, None) for t in range(args.warmup, n_steps)],
                             args.steps)
    # Pass 4: the same timed steps from the same state, each after a cache scrub.
    reset()
    for t in range(args.warmup):
        step(t)
    scrub_step_ms = scrubbed_ms(lambda i: step(args.warmup + i), args.steps, stream)

    def timed(fn, n):
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(n):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    si, so = o["state"][cur[0]], o["state"][1 - cur[0]]
    # Stages replayed from a captured graph: the chunk scores are three short
    # launches, which back-to-back calls from the host cannot keep fed.
    stages = {
        "chunk_scores": graph_ms(lambda: [api.kvc_wnw_chunk_scores(spec, prm, qs[-1], k,
                                                                   o["sigma"], o["ws"])
                                          for _ in range(args.steps)], args.steps),
        "update": graph_ms(lambda: [api.kvc_wnw_update(spec, prm, o["sigma"], si, so)
                                    for _ in range(args.steps)], args.steps),
    }
    # Cold step: from the empty state, every selected block is recalled.
    cold = []
    for _ in range(max(3, args.steps // 4)):
        reset()
        torch.cuda.synchronize()
        ev0.record(stream)
        step(0)
        ev1.record(stream)
        torch.cuda.synchronize()
        cold.append(ev0.elapsed_time(ev1))
    V = api.WnwViews(spec, prm, lay, o["state"][cur[0]])
    cold_rows = 0
    for i, n in enumerate(cfg.lens):
        rb = V.recalled_block[i].cpu().numpy()
        for r in range(int(V.n_recalled[i].item())):
            cold_rows += min(S, int(n) - int(rb[r]) * S)
    cold_ms = sorted(cold)[len(cold) // 2]
    # the recall alone on the cold step's list
    so_cold = o["state"][cur[0]]
    recall_ms = timed(lambda i: api.kvc_wnw_recall(spec, prm, so_cold, hk, hv, o["slot_k"],
                                                   o["slot_v"], stream), args.steps)
    cold_bytes = cold_rows * row_bytes
    recall_gbs = cold_bytes / (recall_ms * 1e-3) / 1e9
    anchor_bytes = sum(int(n) for n in cfg.lens) * int(lay.n_anchor) * d * 2
    score_gbs = anchor_bytes / (stages["chunk_scores"] * 1e-3) / 1e9
    log(f"[bench] wnw step {step_ms * 1e3:.1f} us ({graph_step_ms * 1e3:.1f} us from a graph, "
        f"{scrub_step_ms * 1e3:.1f} us after a cache scrub), "
        f"{bytes_per_step / 1e6:.3f} MB recalled per "
        f"step; chunk scores {stages['chunk_scores'] * 1e3:.1f} us, update "
        f"{stages['update'] * 1e3:.1f} us (stages from a graph); cold step {cold_ms * 1e3:.1f} us recalling "
        f"{cold_bytes / 1e6:.2f} MB ({recall_gbs:.1f} GB/s in the recall kernel)")
    out = {
        "workload": f"{cfg.name}: {cfg.n_seq} seq x n={list(cfg.lens)} audio tokens, "
                    f"{cfg.n_layers} layers x {cfg.n_kv_heads} KV heads ({lay.n_anchor} anchor, "
                    f"{lay.n_tidal} tidal), GQA {cfg.gqa}, head_dim {d}, bf16; chunks "
                    f"{prm.chunk_len}/{prm.chunk_stride} tokens, top {prm.top_chunks}, release "
                    f"after {prm.release_after}",
        "us_per_step": round(step_ms * 1e3, 2),
        "us_per_step_graph": round(graph_step_ms * 1e3, 2),
        "us_per_step_scrubbed": round(scrub_step_ms * 1e3, 2),
        "steps_per_s": 1e3 / step_ms,
        "recalled_bytes_per_step": bytes_per_step,
        "recalled_blocks": [b for b, _ in rec_blocks[args.warmup:]],
        "stage_us": {n2: round(t * 1e3, 2) for n2, t in stages.items()},
        "cold_step_us": round(cold_ms * 1e3, 2),
        "cold_recall_bytes": cold_bytes,
        "roofline": {
            "recall": {"bound": "pcie", "kernel": f"wnw_recall_kernel<{d}>",
                       "achieved": round(recall_gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                       "frac": round(recall_gbs / PCIE_PEAK_GBS, 4),
                       "note": "cold-step recall list, host to device over PCIe"},
            "chunk_scores": {"bound": "hbm", "kernel": "wnw_logits_kernel + wnw_lse_kernel + wnw_mass_kernel",
                             "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                             "traffic": summed_traffic("wnw.hip", ("wnw_logits_kernel",
                                                                   "wnw_lse_kernel",
                                                                   "wnw_mass_kernel"), cfg.name)},
        },
    }
    if not args.no_cpu_baseline:
        from oracle import wnw as Wo
        n = int(cfg.lens[0])
        ks = [synth.bf16_bits_to_f32(ka[0, a, :n]).astype(np.float64)
              for a in range(len(cfg.anchors))]
        st = Wo.Residency(n, S, prm.chunk_len, prm.top_chunks, prm.release_after)
        t0 = time.perf_counter()
        nst = 5
        for t in range(nst):
            qa = synth.bf16_bits_to_f32(synth.wnw_queries(cfg, t, ka)[0]).astype(np.float64)
            _, _, st, _ = Wo.step(st, list(qa), ks)
        ts = (time.perf_counter() - t0) / nst
        out["cpu_baseline"] = dict(value=1.0 / ts, unit="steps/s (scores + update, no copies)",
                                   cores=1, kind="oracle",
                                   sample=f"{nst} decode steps of sequence 0 of the same workload, "
                                          f"{ts * 1e3:.1f} ms per step")
    del hk, hv, k
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="omni30b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step (decayed eviction) measurement")
    ap.add_argument("--decode-config", default="vz_omni30b")
    ap.add_argument("--no-c3", action="store_true",
                    help="skip the query-guided retrieval (C3) measurement")
    ap.add_argument("--c3-config", default="c3_omni30b")
    ap.add_argument("--c3-builds", type=int, default=3)
    ap.add_argument("--c3-only", action="store_true",
                    help="measure only the C3 leg and print its object")
    ap.add_argument("--no-wnw", action="store_true",
                    help="skip the chunk-recall (WnW) measurement")
    ap.add_argument("--wnw-config", default="wnw_voxtral3b")
    ap.add_argument("--wnw-only", action="store_true",
                    help="measure only the WnW leg and print its object")
    ap.add_argument("--power-sample", type=float, default=0.0, metavar="SECONDS",
                    help="after the stage timings, loop the two score passes, the gather "
                         "and the whole step for SECONDS each and log amd-smi's socket "
                         "power and shader clocks")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    # The collector stays off while launches are timed: a full collection
    # pausing the host for tens of ms inside a timed loop leaves the GPU idle
    # and shows up as kernel time.  Each leg collects once before it starts.
    gc.disable()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by (sequence, layer, KV head) unit with no exchange; "
              "multi-GPU runs are out of scope here)", file=sys.stderr)
        sys.exit(2)

    import torch
    from audio_kv_cache_amd import api, synth

    if args.c3_only:
        print(json.dumps(bench_c3(args)), flush=True)
        return
    if args.wnw_only:
        print(json.dumps(bench_wnw(args)), flush=True)
        return

    cfg = synth.CONFIGS[args.config]
    log(f"[bench] generating {cfg.name} inputs")
    t0 = time.perf_counter()
    prob = synth.problem(cfg)
    hdr = prob.hdr
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; copying to the GPU")

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v = dev(prob.q), dev(prob.k), dev(prob.v)
    S = torch.from_numpy(hdr.head_scores).cuda()
    units = [(i, l, h) for i in range(cfg.n_seq) for l in range(cfg.n_layers)
             for h in range(cfg.n_kv_heads)]
    del prob
    spec = api.Spec.for_tensors(k, v, gqa=cfg.gqa, seq_lens=hdr.lengths,
                                retention=hdr.retention, n_window=cfg.n_window)
    prm = api.Params(cfg.alpha, cfg.rho, cfg.window, cfg.base_ratio, cfg.budget_pool)
    out = api.allocate(spec, prm, k.device)
    stream = torch.cuda.current_stream()

    def step(st=stream):
        api.kvc_compress(spec, prm, q, k, v, S, out["k_out"], out["v_out"], out["idx"],
                         out["offsets"], out["budgets"], out["workspace"], st)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # the same K steps replayed from one captured graph (no host launches)
    ms_graph = graph_ms(lambda: [step(None) for _ in range(args.steps)], args.steps)
    log(f"[bench] from a graph: {ms_graph:.3f} ms/step")
    # per-step spread: K more steps, each between its own pair of events
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    pct = {f"p{p}": round(float(np.percentile(per_step, p)), 4) for p in (10, 50, 90)}
    budgets = out["budgets"].cpu().numpy()
    ab = algorithmic_bytes(cfg, hdr, budgets)
    tokheads = sum(int(L) for L in hdr.lengths) * cfg.n_layers * cfg.n_kv_heads
    value = tokheads / (ms * 1e-3)
    path_gbs = ab["total"] / (ms * 1e-3) / 1e9
    log(f"[bench] {ms:.3f} ms/step, {value:.4g} tokens·heads/s, path {path_gbs:.0f} GB/s "
        f"({100 * path_gbs / HBM_PEAK_GBS:.1f} % of HBM peak)")

    # A measured ceiling beside the spec peak: a plain 2 GiB device copy
    # (1 GiB read + 1 GiB written), timed with events.
    csrc = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() * 4 * 5 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del csrc, cdst
    log(f"[bench] device copy ceiling {copy_gbs:.0f} GB/s")

    if args.calib_copy:
        # A plain copy of known size: what HBM counters read for it scales
        # the counters of the path's kernels to bytes.
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Per-kernel timing with events on the stream the kernels run on: each
    # stage entry point launches that step's kernels only (kvc_score_stats
    # launches the statistics kernel and the small LSE fold).
    stages = {}
    if not args.no_stages:
        s_rows = torch.empty(spec.score_rows(), dtype=torch.float32, device="cuda")
        sh_rows = torch.empty_like(s_rows)
        kst = torch.empty(spec.n_units, dtype=torch.int32, device="cuda")
        ws = out["workspace"]
        api.kvc_scores(spec, prm, q, k, s_rows, ws, stream)
        api.kvc_smooth(spec, prm, s_rows, sh_rows, kst, stream, ws)
        calls = {
            "budget": lambda: api.kvc_budget(spec, prm, S, out["budgets"], out["offsets"], stream),
            "score_stats": lambda: api.kvc_score_stats(spec, prm, q, k, ws, stream),
            "score_pool": lambda: api.kvc_score_pool(spec, prm, q, k, s_rows, ws, stream),
            "smooth": lambda: api.kvc_smooth(spec, prm, s_rows, sh_rows, kst, stream, ws),
            "select": lambda: api.kvc_select(spec, prm, sh_rows, out["budgets"], out["offsets"],
                                             out["idx"], stream),
            # the fixed heads' segment-wise variant (WnW), 50-position segments
            "select_segments": lambda: api.kvc_wnw_fixed_select(
                spec, prm, 50, sh_rows, out["budgets"], out["offsets"], out["idx"], stream),
            "gather": lambda: api.kvc_gather(spec, prm, k, v, out["idx"], out["offsets"],
                                             out["k_out"], out["v_out"], stream),
        }
        for name, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(args.steps):
                fn()
            ev1.record(stream)
            torch.cuda.synchronize()
            stages[name] = ev0.elapsed_time(ev1) / args.steps
        log("[bench] stage ms: " + ", ".join(f"{n} {t:.3f}" for n, t in stages.items()))
        if args.power_sample > 0:
            pc = {n: calls[n] for n in ("score_stats", "score_pool", "gather")}
            pc["step"] = step
            ms_each = dict(stages, step=ms)
            power_sample(pc, ms_each, args.power_sample, torch.cuda.synchronize)

    # Rooflines.  The dominant kernel is the pooling pass of the scores; its
    # tighter bound is HBM (K must be streamed) unless the MFMA work takes
    # longer at peak.  One launch per sequence; per-launch figures are the
    # step's totals divided by the launches.
    roof, others = None, {}
    if stages:
        launches = cfg.n_seq

        def hbm(name, kernel, nbytes, ms, src):
            gbs = nbytes / (ms * 1e-3) / 1e9
            return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": committed_traffic(src, kernel.split("<")[0], cfg.name),
                    "algorithmic_bytes": nbytes // launches, "avg_launch_us":
                        round(ms * 1e3 / launches, 1),
                    "frac_of_copy": round(gbs / copy_gbs, 4)}

        t_hbm = ab["pool"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = ab["score_flops"] / (MFMA_PEAK_TFLOPS[cfg.dtype] * 1e12)
        pool_kernel = (f"kvc_score_pool_qs_kernel<d={cfg.head_dim}, blocks={cfg.gqa * cfg.n_window // 32}>"
                       if cfg.dtype == "bf16" else "kvc_score_pool_kernel<TF64>")
        # The pooling pass is a contraction whose MFMA work, per-logit VALU
        # work and K stream each need about a third of its time at their
        # peak rates; measured, it is bound by issuing the matrix and vector
        # work (which overlap only in part, at the lower shader clock the
        # part runs under matrix load), not by HBM.  It is reported against
        # the bf16 matrix peak, with the HBM and VALU fractions beside it.
        tf = ab["score_flops"] / (stages["score_pool"] * 1e-3) / 1e12
        h = hbm("score_pool", pool_kernel, ab["pool"], stages["score_pool"], "score.hip")
        roof = {"bound": "mfma", "kernel": pool_kernel, "achieved": round(tf, 2),
                "peak": MFMA_PEAK_TFLOPS[cfg.dtype], "unit": "TFLOP/s",
                "frac": round(tf / MFMA_PEAK_TFLOPS[cfg.dtype], 4), "traffic": h["traffic"],
                "algorithmic_bytes": h["algorithmic_bytes"], "flops": ab["score_flops"] // launches,
                "avg_launch_us": h["avg_launch_us"], "hbm_achieved_gbs": h["achieved"],
                "hbm_frac": h["frac"], "hbm_frac_of_copy": h["frac_of_copy"],
                "time_at_peak_us": {"mfma": round(t_mfma * 1e6 / launches, 1),
                                    "hbm": round(t_hbm * 1e6 / launches, 1)}}
        # Beside HBM and MFMA, the per-element VALU work of both passes: an FMA,
        # an exponential (two FMA issue slots) and an add per logit, against
        # the VALU issue rate (lane-ops/s).
        logits = ab["score_flops"] // (2 * cfg.head_dim)

        def valu_frac(ms):
            return round(4 * logits / (ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4)
        roof["valu_frac"] = valu_frac(stages["score_pool"])
        roof["time_at_peak_us"]["valu"] = round(4 * logits / (VALU_PEAK_TOPS * 1e12) * 1e6
                                                / launches, 1)
        others["score_stats"] = hbm("score_stats", "kvc_score_stats_qs_kernel" if cfg.dtype == "bf16"
                                    else "kvc_score_stats_kernel", ab["stats"],
                                    stages["score_stats"], "score.hip")
        others["score_stats"]["mfma_frac"] = round(
            ab["score_flops"] / (stages["score_stats"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[cfg.dtype], 4)
        others["score_stats"]["valu_frac"] = valu_frac(stages["score_stats"])
        others["gather"] = hbm("gather", "kvc_gather_kernel<256>", ab["gather"], stages["gather"],
                               "gather.hip")

    decode = None if args.no_decode else bench_decode(args)
    retrieval = None if args.no_c3 else bench_c3(args)
    recall = None if args.no_wnw else bench_wnw(args)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of units")
        cpu = cpu_baseline(cfg, hdr, units, budgets)
        log(f"[bench] oracle {cpu['value']:.4g} tokens·heads/s on {cpu['cores']} threads "
            f"({cpu['one_thread_value']:.4g} on one; {cpu['affinity_cores']} usable cores, "
            f"{cpu['cpu_model']})")

    line = {
        "metric": "compressed tokens·heads/s and % of HBM peak, L=32K audio tokens, 1 GPU",
        "value": value, "unit": "tokens·heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_graph": round(ms_graph, 4),
        "ms_per_step_percentiles": pct, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_seq} seq x L={int(hdr.lengths[0]) if cfg.n_seq == 1 else 'ragged'}"
                               f", {cfg.n_layers} layers x {cfg.n_kv_heads} KV heads, GQA {cfg.gqa}, "
                               f"head_dim {cfg.head_dim}, {cfg.dtype}, retention "
                               f"{float(hdr.retention[0]) if cfg.n_seq == 1 else 'U(0.2,0.6)'}, "
                               f"alpha {cfg.alpha}, rho {cfg.rho}, w {cfg.window}",
                   "tokens_heads_per_step": tokheads,
                   "algorithmic_bytes_per_step": ab["total"]},
        "path_hbm": {"achieved": round(path_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(path_gbs / HBM_PEAK_GBS, 4),
                     "copy_ceiling": round(copy_gbs, 1),
                     "frac_of_copy": round(path_gbs / copy_gbs, 4)},
        "stage_ms": {k2: round(v2, 4) for k2, v2 in stages.items()},
        "roofline": roof,
        "roofline_other_kernels": others,
        "decode": decode,
        "retrieval": retrieval,
        "recall": recall,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
