"""dcut_allocate on the GPU is bit-exact with the oracle given the same fp32
confidences: random, tie-heavy, underflowing (denormal) products, ragged and
invalid max_depth, budgets from B to beyond sum K_b, and the largest B*K."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def run(conf, budget, max_depth=None):
    import draft_verification_verify_amd as sv
    d = sv.dcut_allocate(dev(conf), budget, dev(max_depth))
    torch.cuda.synchronize()
    return host(d)


def test_dcut_random_bit_exact():
    g = np.random.default_rng(31)
    for trial in range(60):
        B = int(g.integers(1, 130))
        K = int(g.integers(1, 20))
        conf = g.uniform(0.0, 1.0, (B, K)).astype(np.float32)
        if trial % 4 == 0:
            conf = np.round(conf * 3) / 3
        if trial % 5 == 0:
            conf[g.random((B, K)) < 0.1] = np.nan
        kb = g.integers(0, K + 1, B).astype(np.int32) if trial % 2 else None
        budget = int(g.integers(B, B * K + 5))
        want = oracle.dcut_allocate(conf, budget, kb)
        got = run(conf, budget, kb)
        assert np.array_equal(want, got), (trial, B, K, budget)


def test_dcut_denormal_products_and_ties():
    B, K = 40, 16
    conf = np.full((B, K), 1e-3, np.float32)
    conf[::3] = 2e-3
    conf[5, :] = 1.0
    for budget in (B, B + 1, 100, 300, B * K, B * K + 100):
        want = oracle.dcut_allocate(conf, budget)
        assert np.array_equal(run(conf, budget), want), budget


def test_dcut_invalid_max_depth_and_largest_batch():
    conf = np.full((4, 5), 0.9, np.float32)
    kb = np.array([5, 6, -1, 0], np.int32)
    assert run(conf, 9, kb).tolist() == oracle.dcut_allocate(conf, 9, kb).tolist() == [5, -1, -1, 0]
    g = np.random.default_rng(7)
    B, K = 2048, 16                      # B*K = 32768, the limit
    conf = g.uniform(0.2, 1.0, (B, K)).astype(np.float32)
    for budget in (B, 9000, B * K):
        assert np.array_equal(run(conf, budget), oracle.dcut_allocate(conf, budget))


def test_dcut_config_sizes():
    # the two workload budgets: B=64,K=16 budget 384; B=64 mixed K_b in {3,16} budget 512
    g = np.random.default_rng(3)
    conf = g.uniform(0.001, 0.3, (64, 16)).astype(np.float32)
    assert np.array_equal(run(conf, 384), oracle.dcut_allocate(conf, 384))
    kb = np.where(g.random(64) < 0.5, 3, 16).astype(np.int32)
    assert np.array_equal(run(conf, 512, kb), oracle.dcut_allocate(conf, 512, kb))


# ------------------------------------------------------- cost-aware D-cut ----

def _rand_table(g, n):
    t = np.cumsum(g.uniform(0.5, 4.0, n))
    c = np.cumsum(g.uniform(0.05, 1.0, n))
    return tuple(zip(t.tolist(), c.tolist()))


def _int_table(g, n):
    """Integer table depths, so that integer d lands on table points."""
    t = np.cumsum(g.integers(1, 4, n)).astype(np.float64)
    c = np.cumsum(g.uniform(0.05, 1.0, n))
    return tuple(zip(t.tolist(), c.tolist()))


@pytest.mark.parametrize("B,K", [(1, 1), (5, 3), (64, 16), (300, 64), (4096, 16), (4096, 1024)])
def test_dcut_cost_random_bit_exact(B, K):
    print(f"\n[case] dcut_allocate_cost random B={B} K={K}", flush=True)
    import draft_verification_verify_amd as sv
    g = np.random.default_rng(B * 7 + K)
    for trial in range(4):
        conf = g.uniform(0.0, 1.0, (B, K)).astype(np.float32)
        conf[g.random((B, K)) < 0.05] = np.float32("nan")
        conf[g.random((B, K)) < 0.03] = 1.5
        conf[g.random((B, K)) < 0.03] = 1.0
        md = g.integers(-1, K + 2, B).astype(np.int32) if trial != 1 else None
        table = (oracle.DEFAULT_COST_TABLE if trial == 0 else
                 _int_table(g, int(g.integers(1, 33))) if trial == 3 else _rand_table(g, int(g.integers(1, 33))))
        budget = float(g.uniform(0.0, 3.0 * B))
        want = oracle.dcut_allocate_cost(conf, budget, md, table)
        got = host(sv.dcut_allocate_cost(dev(conf), budget, dev(md), table))
        assert np.array_equal(got, want), (trial, np.nonzero(got != want)[0][:10])


def test_dcut_cost_ties_and_budget_edges():
    print("\n[case] dcut_allocate_cost ties (equal benefits) and budget edges", flush=True)
    import draft_verification_verify_amd as sv
    conf = np.ones((64, 16), np.float32)
    for budget in (0.0, 2.999, 3.0, 96.0, 191.9, 192.0, 1e9):
        want = oracle.dcut_allocate_cost(conf, budget)
        got = host(sv.dcut_allocate_cost(dev(conf), budget))
        assert np.array_equal(got, want), budget
    # equal benefits go in request order
    assert host(sv.dcut_allocate_cost(dev(conf), 9.0)).tolist()[:4] == [16, 16, 16, 0]


# ------------------------------------ GPU confidence -> GPU D-cut, end to end ----

def _prefix_conf(conf, max_depth):
    """fp32 running products of the sanitised confidence (the D-cut rule),
    0 outside each request's window."""
    B, K = conf.shape
    c = np.nan_to_num(conf.astype(np.float32), nan=0.0)
    c = np.clip(c, np.float32(0.0), np.float32(1.0)).astype(np.float32)
    out = np.zeros((B, K), np.float32)
    for b in range(B):
        Kb = K if max_depth is None else int(max_depth[b])
        run = np.float32(1.0)
        for k in range(max(0, min(Kb, K))):
            run = c[b, k] if k == 0 else np.float32(run * c[b, k])
            out[b, k] = run
    return out


def _taken(depth):
    """Entries (b, k), 1 <= k < d_b, that a depth vector takes beyond the floor."""
    return {(b, k) for b, d in enumerate(depth.tolist()) for k in range(1, max(d, 0))}


@pytest.mark.parametrize("name,seed", [("dcut_ragged", 0), ("dcut_ragged", 1), ("dcut_ragged", 2), ("mixed", 0)])
def test_dcut_from_gpu_confidence_end_to_end(name, seed):
    print(f"\n[case] GPU confidence -> GPU dcut_allocate -> ragged sample: {name} seed {seed}", flush=True)
    import draft_verification_verify_amd as sv
    from parity import compare_sample
    w = synth.dcut_ragged(seed, T=1.0) if name == "dcut_ragged" else synth.mixed(seed)
    md = None if name == "dcut_ragged" else w.max_depth
    conf_g = sv.draft_confidence(dev(w.draft), dev(md))
    depth_g = host(sv.dcut_allocate(conf_g, w.budget, dev(md)))
    conf_o = oracle.draft_confidence(w.draft, md)
    depth_o = oracle.dcut_allocate(conf_o, w.budget, md)
    assert int(depth_g.sum()) == int(depth_o.sum())
    c = _prefix_conf(conf_o, md).astype(np.float64)
    extra, missing = _taken(depth_g) - _taken(depth_o), _taken(depth_o) - _taken(depth_g)
    assert len(extra) == len(missing)
    # a difference is allowed only between entries whose prefix confidence
    # (the oracle's) differs by less than 1e-6 relative
    for e in extra:
        for f in missing:
            assert abs(c[e] - c[f]) < 1e-6 * max(c[e], c[f]), (e, f, c[e], c[f])
    # the verify the bench times, on the GPU's own depths
    out, n, p, q = sv.verify_sample(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                    dev(w.u_accept), dev(w.u_sample), dev(depth_g))
    torch.cuda.synchronize()
    compare_sample(w, host(out), host(n), host(p), host(q), depth_g).assert_ok(f"{name} ragged")
