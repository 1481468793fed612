"""GPU parity of spec_verify_greedy / spec_verify_sample / spec_draft_confidence
against the CPU oracle, through the C ABI (the Python binding).

Inputs are the seeded synthetic workloads (synth/): the five workload shapes
at full size, reduced sizes that still span several chunks and a ragged
tail, and shape/edge fuzz (V not a multiple of the vector width, depth 0,
K = 0, ties everywhere, masked tokens, bad data)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import Tally, compare_greedy, compare_sample, dev, host, run_greedy, run_sample, run_sample_reuse

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    import draft_verification_verify_amd  # noqa: F401  (fails loudly if the library is missing)


# ---------------------------------------------------------------- greedy ----

@pytest.mark.parametrize("seed", range(3))
def test_greedy_tiny(seed):
    note(f"greedy tiny seed={seed}")
    w = synth.tiny(seed, T=0.0)
    out, n = run_greedy(w)
    assert len(compare_greedy(w, out, n)) == 0
    # a drafter that always proposes the target argmax is accepted in full
    am = np.argmax(synth.as_f64(w.target), axis=2).astype(np.int32)
    out, n = run_greedy(w, tokens=am[:, :w.K].copy())
    assert np.all(n == w.K) and np.array_equal(out, am)


@pytest.mark.parametrize("dtype,V", [("bf16", 1), ("bf16", 7), ("bf16", 8), ("bf16", 63), ("f32", 64),
                                     ("f32", 1000), ("bf16", 4099), ("f32", 5003), ("bf16", 70001)])
@pytest.mark.parametrize("K", [0, 1, 3, 16])
def test_greedy_fuzz_shapes(dtype, V, K):
    note(f"greedy fuzz {dtype} V={V} K={K}")
    B = 5
    w = synth.random_case(V * 31 + K, B=B, K=K, V=V, dtype=dtype, temps=(0.0,), sigma=0.2)
    g = np.random.default_rng(V + K)
    depth = g.integers(0, K + 1, B).astype(np.int32)
    out, n = run_greedy(w, depth)
    tal = Tally()
    compare_greedy(w, out, n, depth, tal)
    out2, n2 = run_greedy(w)
    compare_greedy(w, out2, n2, None, tal)
    assert not tal.hard, tal.hard


def test_greedy_ties_and_masks():
    note("greedy ties/masks")
    B, K, V = 6, 4, 3000
    g = np.random.default_rng(9)
    z = np.zeros((B, K + 1, V), np.float32)
    z[0] = 1.5                                   # every entry ties: lowest index wins
    z[1] = -np.inf
    z[1, :, 2999] = -3.0                         # only the last token is finite
    z[2] = np.round(g.standard_normal((K + 1, V)) * 2) / 2   # heavy ties
    z[3, :, 0] = -0.0
    z[3, :, 1:] = -1.0                           # -0.0 is the max
    z[3, :, 5] = 0.0                             # +0.0 ties -0.0: index 0 wins
    z[4] = g.standard_normal((K + 1, V))
    z[4, :, ::2] = -np.inf
    z[5] = g.standard_normal((K + 1, V))
    for dt in ("f32", "bf16"):
        t = z if dt == "f32" else synth.to_bf16_bits(z)
        vals = synth.as_f64(t)
        am = np.argmax(vals, axis=2).astype(np.int32)
        tok = am[:, :K].copy()
        tok[5, 2] = (tok[5, 2] + 1) % V
        w = synth.Workload("ties", dt, t, t[:, :K], tok, np.zeros(B, np.float32),
                           np.zeros((B, K), np.float32), np.zeros(B, np.float32), np.full(B, K, np.int32))
        out, n = run_greedy(w)
        assert len(compare_greedy(w, out, n)) == 0
        assert out[0].tolist() == [0] * (K + 1)
        assert out[1].tolist() == [2999] * (K + 1)
        assert out[3, 0] == 0 and n[5] == 2


def test_greedy_bad_inputs():
    note("greedy bad inputs")
    B, K, V = 6, 3, 777
    w = synth.random_case(3, B=B, K=K, V=V, dtype="f32", temps=(0.0,), sigma=0.1)
    t = w.target.copy()
    tok = w.tokens.copy()
    tok[0, 1] = V
    t[1, 2, 5] = np.nan
    t[2, 3, :] = np.nan          # outside depth-2 window: fine
    t[3, 0, :] = -np.inf
    t[4, 1, 100] = np.inf
    depth = np.array([3, 3, 2, 3, 3, 3], np.int32)
    w2 = synth.Workload("bad", "f32", t, w.draft, tok, w.temperature, w.u_accept, w.u_sample, w.max_depth)
    out, n = run_greedy(w2, depth)
    assert len(compare_greedy(w2, out, n, depth)) == 0
    assert n.tolist()[:2] == [-1, -1] and n[2] >= 0 and n[3] == -1 and n[4] == -1 and n[5] >= 0
    depth2 = np.array([4, -1, 2, 3, 3, 3], np.int32)
    out, n = run_greedy(w2, depth2)
    assert n[0] == -1 and n[1] == -1 and np.all(out[:2] == -1)


@pytest.mark.parametrize("name", ["mtp_chat", "block_code", "dcut_ragged"])
def test_greedy_workloads_full_size(name):
    note(f"greedy full-size {name}")
    w = getattr(synth, name)(0, T=0.0)
    out, n = run_greedy(w)
    assert len(compare_greedy(w, out, n)) == 0
    assert n.mean() > 0


def test_greedy_mixed_fp32_full_size():
    note("greedy mixed fp32 B=64 V=152064 (depth = K_b; padding rows are NaN)")
    w = synth.mixed(0)
    depth = w.max_depth.copy()
    out, n = run_greedy(w, depth)
    assert len(compare_greedy(w, out, n, depth)) == 0
    assert np.all(n >= 0)


# --------------------------------------------------------------- sampled ----

def test_sample_tiny_many_seeds():
    note("sample tiny: 1024 seeded requests of V=1000 at T=1 and T=0")
    tal = Tally()
    for T in (1.0, 0.0):
        ws = [synth.tiny(s, T=T) for s in range(256)]
        w = synth.Workload("tiny_batch", "f32", np.concatenate([x.target for x in ws]),
                           np.concatenate([x.draft for x in ws]), np.concatenate([x.tokens for x in ws]),
                           np.concatenate([x.temperature for x in ws]), np.concatenate([x.u_accept for x in ws]),
                           np.concatenate([x.u_sample for x in ws]), np.concatenate([x.max_depth for x in ws]))
        out, n, p, q = run_sample(w)
        compare_sample(w, out, n, p, q, tally=tal)
    tal.assert_ok("tiny")


@pytest.mark.parametrize("dtype,V", [("bf16", 1), ("f32", 7), ("bf16", 8), ("f32", 63), ("bf16", 64),
                                     ("f32", 1000), ("bf16", 4099), ("f32", 9001), ("bf16", 70001)])
@pytest.mark.parametrize("K", [0, 1, 3, 16])
def test_sample_fuzz_shapes(dtype, V, K):
    note(f"sample fuzz {dtype} V={V} K={K}")
    B = 6
    w = synth.random_case(V * 7 + K, B=B, K=K, V=V, dtype=dtype, temps=(0.0, 0.7, 1.0, 1.6), sigma=0.6)
    g = np.random.default_rng(V * 3 + K)
    depth = g.integers(0, K + 1, B).astype(np.int32)
    tal = Tally()
    out, n, p, q = run_sample(w, depth)
    compare_sample(w, out, n, p, q, depth, tal)
    out, n, p, q = run_sample(w)
    compare_sample(w, out, n, p, q, None, tal)
    tal.assert_ok(f"{dtype} V={V} K={K}")


def test_sample_bad_inputs():
    note("sample bad inputs")
    w = synth.random_case(1, B=8, K=3, V=640, dtype="f32", temps=(1.0,))
    t, d = w.target.copy(), w.draft.copy()
    tok, ua, us, T = w.tokens.copy(), w.u_accept.copy(), w.u_sample.copy(), w.temperature.copy()
    depth = np.array([3, 3, 3, 1, 3, 3, 3, 3], np.int32)
    tok[0, 2] = -1
    ua[1, 0] = 1.0
    T[2] = -0.5
    d[3, 2, :] = np.nan
    d[4, 1, 3] = np.nan
    T[5] = np.nan
    us[6] = 1.5
    t[7, 3, :] = -np.inf         # bonus row: bad only if it is read (no rejection)
    w2 = synth.Workload("bad", "f32", t, d, tok, T, ua, us, w.max_depth)
    out, n, p, q = run_sample(w2, depth)
    tal = compare_sample(w2, out, n, p, q, depth)
    tal.assert_ok("bad inputs")
    assert n.tolist()[:3] == [-1, -1, -1] and n[4] == -1 and n[5] == -1 and n[6] == -1
    assert n[3] >= 0


@pytest.mark.parametrize("name,kw", [("mtp_chat", {}), ("mtp_chat", {"literal": True}),
                                     ("block_code", {}), ("block_code", {"boost": 14.0}),
                                     ("dcut_ragged", {})])
def test_sample_workloads_full_size(name, kw):
    note(f"sample full-size {name} {kw}")
    tal = Tally()
    for seed in range(2):
        w = getattr(synth, name)(seed, T=1.0, **kw)
        out, n, p, q = run_sample(w)
        compare_sample(w, out, n, p, q, tally=tal)
    tal.assert_ok(name)


def test_dcut_pipeline_full_size():
    note("dcut pipeline B=64 K=16 V=128000: confidence -> dcut_allocate(384) -> ragged sample")
    import draft_verification_verify_amd as sv
    w = synth.dcut_ragged(0, T=1.0)
    conf_g = host(sv.draft_confidence(dev(w.draft)))
    conf_o = oracle.draft_confidence(w.draft)
    assert np.max(np.abs(conf_g - conf_o) / conf_o) < 2e-6
    depth_g = host(sv.dcut_allocate(dev(conf_o), w.budget))
    depth_o = oracle.dcut_allocate(conf_o, w.budget)
    assert np.array_equal(depth_g, depth_o)
    assert int(depth_o.sum()) == w.budget and depth_o.min() >= 1 and depth_o.max() <= w.K
    out, n, p, q = run_sample(w, depth_o)
    tal = compare_sample(w, out, n, p, q, depth_o)
    tal.assert_ok("ragged")


def test_mixed_fp32_pipeline_full_size():
    note("mixed fp32 B=64 V=152064: per-request K_b and T, dcut_allocate(512), one sample launch")
    import draft_verification_verify_amd as sv
    w = synth.mixed(0)
    conf_o = oracle.draft_confidence(w.draft, w.max_depth)
    conf_g = host(sv.draft_confidence(dev(w.draft), dev(w.max_depth)))
    m = conf_o > 0
    assert np.all(conf_g[~m] == 0) and np.max(np.abs(conf_g[m] - conf_o[m]) / conf_o[m]) < 2e-6
    depth = oracle.dcut_allocate(conf_o, w.budget, w.max_depth)
    assert np.array_equal(host(sv.dcut_allocate(dev(conf_o), w.budget, dev(w.max_depth))), depth)
    out, n, p, q = run_sample(w, depth)
    tal = compare_sample(w, out, n, p, q, depth)
    tal.assert_ok("mixed")
    assert np.all(n >= 0)


# ---------------------------------------------- draft-statistics reuse ----

def test_reuse_pipeline_full_size():
    note("reuse pipeline B=64 K=16 V=128000: confidence + row statistics -> dcut_allocate(384) -> sample_reuse")
    import draft_verification_verify_amd as sv
    w = synth.dcut_ragged(0, T=1.0)
    conf_g, st = sv.draft_confidence_stats(dev(w.draft))
    conf_o = oracle.draft_confidence(w.draft)
    assert np.max(np.abs(host(conf_g) - conf_o) / conf_o) < 2e-6
    mx, sm, tt = (host(t) for t in sv.row_stat_fields(st))
    assert np.all(tt == 1.0)
    # the statistics are the rows' maxima and softmax normalisers at T = 1
    assert np.array_equal(mx, synth.as_f64(w.draft).max(axis=2).astype(np.float32))
    assert np.max(np.abs(1.0 / sm - conf_o) / conf_o) < 2e-6
    depth = oracle.dcut_allocate(conf_o, w.budget)
    out, n, p, q = sv.verify_sample_reuse(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                          dev(w.u_accept), dev(w.u_sample), st, dev(depth))
    torch.cuda.synchronize()
    tal = compare_sample(w, host(out), host(n), host(p), host(q), depth)
    tal.assert_ok("reuse ragged")
    assert np.all(host(n) >= 0)


def test_reuse_mixed_temperatures_fp32():
    note("reuse mixed fp32 B=64 V=152064: T in {0, 0.7, 1}; only T = 1 requests use the statistics")
    w = synth.mixed(0)
    conf_o = oracle.draft_confidence(w.draft, w.max_depth)
    depth = oracle.dcut_allocate(conf_o, w.budget, w.max_depth)
    out, n, p, q = run_sample_reuse(w, depth, w.max_depth)
    tal = compare_sample(w, out, n, p, q, depth)
    tal.assert_ok("reuse mixed")
    assert np.all(n >= 0)


@pytest.mark.parametrize("dtype,V", [("f32", 7), ("bf16", 64), ("f32", 1000), ("bf16", 4099), ("f32", 9001)])
@pytest.mark.parametrize("K", [1, 3, 16])
def test_reuse_fuzz_shapes(dtype, V, K):
    note(f"reuse fuzz {dtype} V={V} K={K}")
    B = 6
    w = synth.random_case(V * 11 + K, B=B, K=K, V=V, dtype=dtype, temps=(0.0, 0.7, 1.0, 1.0), sigma=0.6)
    g = np.random.default_rng(V * 5 + K)
    depth = g.integers(0, K + 1, B).astype(np.int32)
    tal = Tally()
    out, n, p, q = run_sample_reuse(w, depth)
    compare_sample(w, out, n, p, q, depth, tal)
    out, n, p, q = run_sample_reuse(w)
    compare_sample(w, out, n, p, q, None, tal)
    tal.assert_ok(f"reuse {dtype} V={V} K={K}")


def test_reuse_depth_beyond_statistics_is_bad():
    note("reuse: a depth past the confidence pass's max_depth is bad data; the rest still verify")
    w = synth.random_case(77, B=4, K=3, V=1000, dtype="f32", temps=(1.0,))
    max_depth = np.array([3, 1, 3, 0], np.int32)
    depth = np.array([3, 2, 1, 0], np.int32)
    out, n, p, q = run_sample_reuse(w, depth, max_depth)
    assert n[1] == -1 and np.all(out[1] == -1)
    ok = np.array([0, 2, 3])
    sub = synth.Workload(w.name, w.dtype, w.target[ok], w.draft[ok], w.tokens[ok], w.temperature[ok],
                         w.u_accept[ok], w.u_sample[ok], w.max_depth[ok])
    tal = compare_sample(sub, out[ok], n[ok], p[ok], q[ok], depth[ok])
    tal.assert_ok("reuse partial")


@pytest.mark.parametrize("B", [65, 66, 129, 300, 4096])
def test_ragged_large_batches_with_empty_requests(B):
    # Each row-pass task finds its request among the plan's row offsets: one
    # ballot round over 64 offsets up to B = 65, two beyond.  Requests with no
    # rows (depth 0 on greedy rows aside, bad temperatures, NaN) leave runs of
    # equal offsets that must never be chosen.
    note(f"ragged batch B={B}: depths in [0, K] with many zeros, bad temperatures, greedy and sampled")
    K, V = 4, 37
    g = np.random.default_rng(B)
    temps = g.choice(np.array([0.0, 0.7, 1.0, 1.0, np.nan], np.float32), B).astype(np.float32)
    w = synth.random_case(B + 17, B=B, K=K, V=V, dtype="f32" if B % 2 else "bf16", temperature=temps, sigma=0.6)
    depth = g.integers(0, K + 1, B).astype(np.int32)
    depth[g.random(B) < 0.3] = 0
    depth[g.random(B) < 0.05] = -1   # bad depth: no rows either
    out, n, p, q = run_sample(w, depth)
    compare_sample(w, out, n, p, q, depth).assert_ok(f"ragged B={B}")
    og, ng = run_greedy(w, depth)
    assert compare_greedy(w, og, ng, depth).size == 0


def test_determinism_and_workspace_reuse():
    note("determinism: repeated calls, shared workspace across shapes")
    import draft_verification_verify_amd as sv
    ws = torch.full((sv.workspace_size(64, 16, 152064),), 0xA5, dtype=torch.uint8, device="cuda")  # garbage
    a = synth.block_code(3, T=1.0, B=6, V=50000)
    b = synth.tiny(4, T=1.0)
    args = lambda w: (dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature), dev(w.u_accept),
                      dev(w.u_sample))
    ra = [tuple(host(x) for x in sv.verify_sample(*args(a), workspace=ws)) for _ in range(2)]
    rb = tuple(host(x) for x in sv.verify_sample(*args(b), workspace=ws))
    ra.append(tuple(host(x) for x in sv.verify_sample(*args(a), workspace=ws)))
    g1 = host(sv.verify_greedy(dev(a.target), dev(a.tokens), workspace=ws)[0])
    g2 = host(sv.verify_greedy(dev(a.target), dev(a.tokens), workspace=ws)[0])
    torch.cuda.synchronize()
    for r in ra[1:]:
        for x, y in zip(ra[0], r):
            assert np.array_equal(x, y)
    assert np.array_equal(g1, g2)
    compare_sample(b, *rb).assert_ok("reuse")


# -------------------------------------------------------- statistics pins ----

def test_lossless_monte_carlo_gpu():
    note("lossless MC on the GPU: V=5, K=3, 200000 requests, chi-square per position")
    from scipy.stats import chisquare
    g = np.random.default_rng(12)
    V, K, B, T = 5, 3, 200000, 1.0
    zrows = (g.standard_normal((K + 1, V)) * 1.3).astype(np.float32)
    yrows = (zrows[:K] + g.standard_normal((K, V)) * 0.9).astype(np.float32)
    target = np.ascontiguousarray(np.broadcast_to(zrows[None], (B, K + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(yrows[None], (B, K, V)))
    tokens = np.empty((B, K), np.int32)
    for k in range(K):
        gum = -np.log(-np.log(g.random((B, V))))
        tokens[:, k] = np.argmax(yrows[k].astype(np.float64)[None] / T + gum, axis=1)
    w = synth.Workload("mc", "f32", target, draft, tokens, np.full(B, T, np.float32),
                       g.random((B, K), dtype=np.float32), g.random(B, dtype=np.float32), np.full(B, K, np.int32))
    import draft_verification_verify_amd as sv
    out = n = None
    for lo in range(0, B, 4096):
        sl = slice(lo, min(B, lo + 4096))
        part = synth.Workload("mc", "f32", w.target[sl], w.draft[sl], w.tokens[sl], w.temperature[sl],
                              w.u_accept[sl], w.u_sample[sl], w.max_depth[sl])
        o, nn, _, _ = run_sample(part)
        out = o if out is None else np.concatenate([out, o])
        n = nn if n is None else np.concatenate([n, nn])
    p = torch.softmax(torch.from_numpy(zrows.astype(np.float64)) / T, dim=1).numpy()
    for k in range(K + 1):
        emitted = out[n >= k, k]
        obs = np.bincount(emitted, minlength=V)
        assert chisquare(obs, p[k] * emitted.size).pvalue > 1e-3
    # and the GPU agrees with the oracle request by request
    sl = slice(0, 4096)
    part = synth.Workload("mc", "f32", w.target[sl], w.draft[sl], w.tokens[sl], w.temperature[sl],
                          w.u_accept[sl], w.u_sample[sl], w.max_depth[sl])
    compare_sample(part, out[sl], n[sl], None, None).assert_ok("mc")


def test_planted_alpha_gpu():
    note("planted acceptance rates on the GPU: E[n] = sum_k prod_{j<=k} alpha_j")
    alphas = [0.81, 0.66, 0.52]
    B = 4000
    w = synth.planted_alpha(1, B, alphas, V=12)
    out, n, p, q = run_sample(w)
    expect = sum(np.prod(alphas[:k + 1]) for k in range(len(alphas)))
    assert abs(n.mean() - expect) < 5 * n.std() / np.sqrt(B)
    compare_sample(w, out, n, p, q).assert_ok("planted")
