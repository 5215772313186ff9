"""GPU parity of C3 query-guided retrieval against the oracle (oracle/c3.py),
through the C ABI of include/kvc_c3.h.

Criteria:
  * tree (index) per cache: node records, node count, member order and
    centroid bits equal to the oracle's, bit for bit (every split decision
    is defined to be reproducible);
  * initial frontier and EMA state: equal;
  * sigma: |sigma - sigma_ref| <= 3e-5 (fp32 dot products of bf16 values
    against the oracle's fp64 cosines, which lie in [-1, 1]);
  * selection and update taken on the GPU's own sigma: kept positions,
    frontier ids and EMA values equal to the oracle's decisions on the same
    sigma;
  * the one-call step equals the stage calls; its K, V rows are K[idx],
    V[idx].
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from audio_kv_cache_amd import _lib as C  # noqa: E402
from audio_kv_cache_amd import api, synth  # noqa: E402
from oracle import c3 as C3  # noqa: E402

pytestmark = pytest.mark.gpu

SIGMA_TOL = 3e-5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


class C3Dev:
    def __init__(self, cfg: synth.C3Config, k=None, v=None, params=None):
        self.cfg = cfg
        if k is None:
            k, v = synth.c3_problem(cfg)
        self.k_np, self.v_np = k, v
        self.k = torch.from_numpy(k.view(np.int16)).cuda().view(torch.bfloat16)
        self.v = torch.from_numpy(v.view(np.int16)).cuda().view(torch.bfloat16)
        self.spec = api.C3Spec(n_layers=cfg.n_layers, n_kv_heads=cfg.n_kv_heads, gqa=cfg.gqa,
                               head_dim=cfg.head_dim, lens=cfg.lens, budgets=cfg.budgets,
                               capacity=cfg.capacity)
        self.params = params or api.C3Params()
        self.o = api.c3_allocate(self.spec, self.params, "cuda")
        self.cur = 0

    @property
    def U(self):
        return self.spec.n_units

    def n_of(self, u):
        return int(self.cfg.lens[u // (self.cfg.n_layers * self.cfg.n_kv_heads)])

    def b_of(self, u):
        return int(self.cfg.budgets[u // (self.cfg.n_layers * self.cfg.n_kv_heads)])

    def build(self):
        o = self.o
        api.kvc_c3_build(self.spec, self.params, self.k, o["index"], o["state"][0], o["build_ws"])
        torch.cuda.synchronize()
        self.cur = 0

    def views(self, which=None):
        s = self.o["state"][self.cur if which is None else which]
        return api.C3Views(self.spec, self.o["layout"], self.o["index"], s)

    def tree(self, u):
        """The GPU's tree of cache u as numpy arrays."""
        V = self.views()
        nn = int(V.n_nodes[u].item())
        n = self.n_of(u)
        g = lambda t: t[u, :nn].cpu().numpy().astype(np.int64)
        return dict(n_nodes=nn, start=g(V.start), size=g(V.size), left=g(V.left),
                    parent=g(V.parent), depth=g(V.depth),
                    centroid=V.centroid[u, :nn].cpu().numpy().view(np.uint16),
                    perm=V.perm[u, :n].cpu().numpy().astype(np.int64))

    def state(self, u, which=None):
        V = self.views(which)
        A = int(V.count[u].item())
        return V.frontier[u, :A].cpu().numpy().astype(np.int64), V.ema[u, :A].cpu().numpy()

    def keys(self, u):
        return bf16_values(self.k_np[u, :self.n_of(u)])


def oracle_tree(dev: C3Dev, u):
    return C3.build_tree(dev.keys(u), cache=u, seed=dev.params.seed)


def centroid_bits(t: C3.Tree) -> np.ndarray:
    return (t.centroid.view(np.uint32) >> 16).astype(np.uint16)


def assert_tree_equal(dev: C3Dev, u, t: C3.Tree):
    g = dev.tree(u)
    assert g["n_nodes"] == t.n_nodes, (u, g["n_nodes"], t.n_nodes)
    for f in ("start", "size", "left", "parent", "depth"):
        assert np.array_equal(g[f], getattr(t, f)), (u, f)
    assert np.array_equal(g["perm"], t.perm), (u, "perm")
    assert np.array_equal(g["centroid"], centroid_bits(t)), (u, "centroid")


def built(name):
    dev = C3Dev(synth.C3_CONFIGS[name])
    say(f"[c3] build {name}")
    dev.build()
    return dev


@pytest.fixture(scope="module")
def mixed():
    return built("c3_mixed")


@pytest.mark.parametrize("name", ["c3_tiny", "c3_mixed", "c3_edge"])
def test_tree_and_initial_frontier_bit_exact(name):
    dev = built(name)
    for u in range(dev.U):
        t = oracle_tree(dev, u)
        assert_tree_equal(dev, u, t)
        F, e = dev.state(u)
        assert np.array_equal(F, C3.initial_frontier(t, dev.n_of(u))), u
        assert (e == 0).all()


def test_build_is_deterministic(mixed):
    lay = mixed.o["layout"]
    index0 = mixed.o["index"].clone()
    state0 = mixed.o["state"][0].clone()
    mixed.build()
    V0 = api.C3Views(mixed.spec, lay, index0, state0)
    V1 = mixed.views()
    for u in range(mixed.U):
        nn = int(V1.n_nodes[u].item())
        assert nn == int(V0.n_nodes[u].item())
        for a, b in ((V0.start, V1.start), (V0.size, V1.size), (V0.left, V1.left),
                     (V0.parent, V1.parent), (V0.depth, V1.depth), (V0.centroid, V1.centroid)):
            assert torch.equal(a[u, :nn], b[u, :nn])
        assert torch.equal(V0.perm[u], V1.perm[u])


def run_steps(dev: C3Dev, steps: int, trees):
    """Stage calls checked against the oracle on the GPU's sigma, then the
    one-call step checked against the stage calls; the state advances."""
    o = dev.o
    for s in range(steps):
        q_np = synth.c3_queries(dev.cfg, s)
        q = torch.from_numpy(q_np.view(np.int16)).cuda().view(torch.bfloat16)
        say(f"[c3] {dev.cfg.name} step {s}")
        sin, sout = o["state"][dev.cur], o["state"][1 - dev.cur]
        o["sigma"].fill_(float("nan"))
        api.kvc_c3_score(dev.spec, dev.params, o["index"], sin, q, o["sigma"])
        idx_stage = torch.full_like(o["idx"], -7)
        api.kvc_c3_select(dev.spec, dev.params, o["index"], sin, o["sigma"], idx_stage)
        api.kvc_c3_update(dev.spec, dev.params, o["index"], sin, o["sigma"], sout)
        torch.cuda.synchronize()
        sig_all = o["sigma"].cpu().numpy()
        idx_all = idx_stage.cpu().numpy()
        upd = [dev.state(u, 1 - dev.cur) for u in range(dev.U)]
        for u in range(dev.U):
            n, B = dev.n_of(u), dev.b_of(u)
            F, e = dev.state(u)
            t = trees[u]
            if n <= B:
                assert idx_all[u, :n].tolist() == list(range(n))
                assert np.array_equal(upd[u][0], F) and np.array_equal(upd[u][1], e)
                continue
            sig = sig_all[u, :len(F)].astype(np.float64)
            ref = C3.node_scores(t, F, bf16_values(q_np[u]))
            err = np.abs(sig - ref).max()
            assert err <= SIGMA_TOL, (u, err)
            kept = C3.retrieve(t, F, sig, n, B)
            assert np.array_equal(idx_all[u, :B], kept), u
            F2, e2 = C3.update_frontier(t, F, e, sig, dev.params.lam, dev.params.r_swaps)
            assert np.array_equal(upd[u][0], F2), u
            assert np.array_equal(upd[u][1], e2), u
        # one call: same decisions, gathered rows
        st2 = torch.empty_like(sout)
        api.kvc_c3_step(dev.spec, dev.params, o["index"], sin, st2, q, dev.k, dev.v,
                        o["k_out"], o["v_out"], o["idx"], o["step_ws"])
        torch.cuda.synchronize()
        lay = o["layout"]
        V2 = api.C3Views(dev.spec, lay, o["index"], st2)
        idx_one = o["idx"].cpu().numpy()
        ko = o["k_out"].view(torch.int16).cpu().numpy().view(np.uint16)
        vo = o["v_out"].view(torch.int16).cpu().numpy().view(np.uint16)
        for u in range(dev.U):
            kn = min(dev.n_of(u), dev.b_of(u))
            assert np.array_equal(idx_one[u, :kn], idx_all[u, :kn]), u
            A = int(V2.count[u].item())
            assert np.array_equal(V2.frontier[u, :A].cpu().numpy(), upd[u][0]), u
            assert np.array_equal(V2.ema[u, :A].cpu().numpy(), upd[u][1]), u
            rows = idx_one[u, :kn]
            assert np.array_equal(ko[u, :kn], dev.k_np[u, rows]), u
            assert np.array_equal(vo[u, :kn], dev.v_np[u, rows]), u
        dev.cur = 1 - dev.cur


@pytest.mark.parametrize("name", ["c3_tiny", "c3_mixed", "c3_edge"])
def test_steps_against_oracle(name):
    dev = built(name)
    trees = [oracle_tree(dev, u) for u in range(dev.U)]
    run_steps(dev, 4, trees)


def test_equal_scores_follow_start_order(mixed):
    # sigma all equal: ranking, splits and merges fall back to start order.
    dev = mixed
    o = dev.o
    trees = [oracle_tree(dev, u) for u in range(dev.U)]
    sin, sout = o["state"][dev.cur], o["state"][1 - dev.cur]
    sig = torch.zeros_like(o["sigma"])
    idx = torch.full_like(o["idx"], -7)
    api.kvc_c3_select(dev.spec, dev.params, o["index"], sin, sig, idx)
    api.kvc_c3_update(dev.spec, dev.params, o["index"], sin, sig, sout)
    torch.cuda.synchronize()
    for u in range(dev.U):
        n, B = dev.n_of(u), dev.b_of(u)
        if n <= B:
            continue
        F, e = dev.state(u)
        z = np.zeros(len(F))
        assert np.array_equal(idx.cpu().numpy()[u, :B], C3.retrieve(trees[u], F, z, n, B))
        F2, e2 = C3.update_frontier(trees[u], F, e, z, dev.params.lam, dev.params.r_swaps)
        Fg, eg = dev.state(u, 1 - dev.cur)
        assert np.array_equal(Fg, F2) and np.array_equal(eg, e2)


@pytest.mark.parametrize("lam,R", [(0.0, 4), (1.0, 1), (0.2, 0)])
def test_other_lambda_and_swaps(lam, R):
    cfg = synth.C3_CONFIGS["c3_tiny"]
    dev = C3Dev(cfg, params=api.C3Params(lam=lam, r_swaps=R, seed=7))
    dev.build()
    trees = [oracle_tree(dev, u) for u in range(dev.U)]
    for u in range(dev.U):
        assert_tree_equal(dev, u, trees[u])
    run_steps(dev, 3, trees)


@pytest.mark.parametrize("gqa,d", [(12, 128), (32, 64), (1, 64)])
def test_group_sizes(gqa, d):
    cfg = synth.C3Config(f"c3_g{gqa}_d{d}", 24, 2, 1, 2, gqa, d, lens=(700, 333),
                         budgets=(64, 40), capacity=704)
    dev = C3Dev(cfg)
    dev.build()
    trees = [oracle_tree(dev, u) for u in range(dev.U)]
    for u in range(dev.U):
        assert_tree_equal(dev, u, trees[u])
    run_steps(dev, 2, trees)


def test_tiny_and_zero_keys_are_snapped_alike():
    # Keys below 2^-17 are moved to the 2^-24 grid before any sum; zeros and
    # subnormal bf16 values as well.
    cfg = synth.C3_CONFIGS["c3_tiny"]
    k, v = synth.c3_problem(cfg)
    r = np.random.default_rng(5)
    tiny = (r.standard_normal((60, cfg.head_dim)) * 3e-6).astype(np.float32)
    tiny[::7] = 0.0
    tiny[3, :5] = np.float32(2.0 ** -130)
    for u in range(k.shape[0]):
        k[u, 100:160] = synth.f32_to_bf16_bits(tiny)
        k[u, 200:210, ::3] = 0
    dev = C3Dev(cfg, k, v)
    dev.build()
    for u in range(dev.U):
        assert_tree_equal(dev, u, oracle_tree(dev, u))


def test_key_out_of_range_is_reported():
    cfg = synth.C3_CONFIGS["c3_tiny"]
    k, v = synth.c3_problem(cfg)
    k[1, 17, 5] = synth.f32_to_bf16_bits(np.array([5000.0], np.float32))[0]
    dev = C3Dev(cfg, k, v)
    with pytest.raises(C.KvcError) as ei:
        dev.build()
    assert ei.value.status == C.KVC_ERR_INVALID_ARG


@pytest.mark.slow
def test_full_size_sampled_caches():
    # The 48-layer, 4-KV-head, 32768-key workload the benchmark times: every
    # cache is built on the GPU; two caches are checked against the oracle's
    # tree and one decode step's decisions.
    dev = built("c3_omni30b")
    sample = [0, dev.U - 1]
    trees = {}
    for u in sample:
        say(f"[c3] oracle tree of cache {u}")
        trees[u] = oracle_tree(dev, u)
        assert_tree_equal(dev, u, trees[u])
        F, e = dev.state(u)
        assert np.array_equal(F, C3.initial_frontier(trees[u], dev.n_of(u)))
    o = dev.o
    q_np = synth.c3_queries(dev.cfg, 0)
    q = torch.from_numpy(q_np.view(np.int16)).cuda().view(torch.bfloat16)
    sin, sout = o["state"][0], o["state"][1]
    api.kvc_c3_step(dev.spec, dev.params, o["index"], sin, sout, q, dev.k, dev.v, o["k_out"],
                    o["v_out"], o["idx"], o["step_ws"])
    sig = torch.empty_like(o["sigma"])
    api.kvc_c3_score(dev.spec, dev.params, o["index"], sin, q, sig)
    torch.cuda.synchronize()
    idx = o["idx"].cpu().numpy()
    for u in sample:
        F, e = dev.state(u, 0)
        s = sig[u, :len(F)].cpu().numpy().astype(np.float64)
        ref = C3.node_scores(trees[u], F, bf16_values(q_np[u]))
        assert np.abs(s - ref).max() <= SIGMA_TOL
        assert np.array_equal(idx[u, :512], C3.retrieve(trees[u], F, s, 32768, 512))
        F2, e2 = C3.update_frontier(trees[u], F, e, s, 0.5, 2)
        Fg, eg = dev.state(u, 1)
        assert np.array_equal(Fg, F2) and np.array_equal(eg, e2)
    # every cache: B distinct ascending positions
    assert (np.diff(idx[:, :512], axis=1) > 0).all()
    assert (idx[:, :512] >= 0).all() and (idx[:, :512] < 32768).all()
