"""Pins for the CPU oracle against what the pages and the mathematics fix.

Each group pins one oracle function with something other than the oracle
itself: closed forms, hand-derived cases, library routines (torch.softmax in
float64, numpy argmax / searchsorted / float32 cumprod), exact enumeration of
the rejection-sampling outcome over stratified uniform grids, planted
acceptance rates with a closed-form mean accepted length, and brute force
over D-cut depth vectors.  A plausible slip in the oracle (a dropped
temperature, a sign flip in the residual, <= for <, the wrong bonus row,
total accepts for first rejection, an off-by-one in the inverse CDF, a
reversed tie rule) fails at least one test here.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def f32(x):
    return np.asarray(x, dtype=np.float32)


def torch_softmax64(row_f64, T):
    return torch.softmax(torch.from_numpy(np.asarray(row_f64, np.float64)) / T, dim=0).numpy()


# --------------------------------------------------------------------------
# softmax
# --------------------------------------------------------------------------

def test_softmax_uniform_closed_form():
    V = 1000
    p, M, S = oracle.softmax(np.full(V, 0.37, np.float32), 1.0)
    assert M == pytest.approx(np.float32(0.37))
    assert S == V                      # every term is exp(0) = 1
    assert np.all(p == 1.0 / V)


@pytest.mark.parametrize("delta,T", [(1.0, 1.0), (2.5, 0.7), (-3.0, 2.0), (0.0, 0.3)])
def test_softmax_two_token_closed_form(delta, T):
    p, _, _ = oracle.softmax(f32([0.0, delta]), T)
    d = float(np.float32(delta))
    assert p[1] == pytest.approx(1.0 / (1.0 + math.exp(-d / T)), rel=1e-15, abs=1e-300)
    assert p[0] + p[1] == pytest.approx(1.0, abs=1e-15)


@pytest.mark.parametrize("T", [0.5, 0.7, 1.0, 2.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_matches_torch_float64(T, dtype):
    g = np.random.default_rng(5)
    z = (g.standard_normal(5000) * 3).astype(np.float32)
    row = synth.to_bf16_bits(z) if dtype == "bf16" else z
    p, _, _ = oracle.softmax(row, T)
    ref = torch_softmax64(synth.as_f64(row), T)
    assert np.max(np.abs(p - ref) / ref) < 1e-12     # rounding order differs (torch scales first)


def test_softmax_masked_entries_and_bad_rows():
    p, _, _ = oracle.softmax(f32([1.0, -np.inf, 2.0, -np.inf]), 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    assert p[2] / p[0] == pytest.approx(math.e, rel=1e-15)
    with pytest.raises(ValueError):
        oracle.softmax(f32([1.0, np.nan, 2.0]), 1.0)
    with pytest.raises(ValueError):
        oracle.softmax(f32([-np.inf, -np.inf]), 1.0)
    with pytest.raises(ValueError):
        oracle.softmax(f32([1.0, np.inf]), 1.0)      # +inf: inf - inf is undefined


# --------------------------------------------------------------------------
# argmax (greedy rule)
# --------------------------------------------------------------------------

def test_argmax_ties_lowest_index():
    assert oracle.argmax(f32([1, 3, 3, 2])) == 1
    assert oracle.argmax(f32([-0.0, 0.0])) == 0
    assert oracle.argmax(f32([0.0, -0.0])) == 0
    assert oracle.argmax(f32([-np.inf, -np.inf, 5.0, 5.0])) == 2
    assert oracle.argmax(f32([7.0])) == 0
    assert oracle.argmax(synth.to_bf16_bits(f32([1.0, 1.001, 1.002]))) == 0  # all round to bf16 1.0


def test_argmax_matches_numpy_on_tie_rich_bf16_rows():
    # N(0, 3^2) rows of 128000 rounded to bf16: a few percent hold a tied max.
    g = np.random.default_rng(11)
    ties = 0
    for _ in range(40):
        row = synth.to_bf16_bits((g.standard_normal(128000) * 3).astype(np.float32))
        vals = synth.as_f64(row)
        ties += int(np.sum(vals == vals.max()) > 1)
        assert oracle.argmax(row) == int(np.argmax(vals))   # numpy: first occurrence
    assert ties >= 1


# --------------------------------------------------------------------------
# inverse CDF
# --------------------------------------------------------------------------

def test_inverse_cdf_matches_searchsorted():
    g = np.random.default_rng(3)
    for _ in range(300):
        V = int(g.integers(1, 60))
        r = g.random(V) * (g.random(V) < 0.7)
        if r.sum() == 0:
            r[0] = 1.0
        u = float(np.float32(g.random()))
        want = int(np.searchsorted(np.cumsum(r), u * r.sum(), side="right"))
        assert oracle.inverse_cdf(r, u) == want


def test_inverse_cdf_boundaries_and_overrun():
    assert oracle.inverse_cdf(np.ones(4), 0.25) == 1        # prefix 1.0 is not > 1.0
    assert oracle.inverse_cdf(np.ones(4), 0.0) == 0
    assert oracle.inverse_cdf(np.array([0.0, 1.0, 0.0, 1.0]), 0.0) == 1   # zero mass never chosen
    assert oracle.inverse_cdf(np.array([0.0, 1.0, 1.0, 0.0, 0.0]), 1.0) == 2  # overrun -> last positive
    assert oracle.inverse_cdf(np.zeros(3), 0.5) == -1


# --------------------------------------------------------------------------
# residual
# --------------------------------------------------------------------------

def test_residual_closed_form_and_fallback():
    t = f32([0, 0, 0, 0])
    d = f32([0, -np.inf, -np.inf, 0])
    r, fb = oracle.residual(t, d, 1.0)
    assert not fb
    assert np.array_equal(r, [0.0, 0.25, 0.25, 0.0])
    r, fb = oracle.residual(t, t, 1.0)        # p == q: no residual mass -> fall back to p
    assert fb and np.array_equal(r, [0.25] * 4)
    r, fb = oracle.residual(f32([0, np.log(3.0)]), None, 1.0)   # bonus: r = p
    assert r == pytest.approx([0.25, 0.75], rel=1e-7)


def test_residual_identity_min_plus_residual_is_p():
    # min(p,q) + (1 - sum min(p,q)) * r/R == p  (the lossless identity)
    g = np.random.default_rng(8)
    for T in (0.7, 1.0, 1.6):
        z = (g.standard_normal(64) * 2).astype(np.float32)
        y = (z + g.standard_normal(64)).astype(np.float32)
        p, _, _ = oracle.softmax(z, T)
        q, _, _ = oracle.softmax(y, T)
        r, fb = oracle.residual(z, y, T)
        assert not fb
        mix = np.minimum(p, q) + (1 - np.minimum(p, q).sum()) * r / r.sum()
        assert np.max(np.abs(mix - p)) < 1e-15


# --------------------------------------------------------------------------
# hand-derived verification cases
# --------------------------------------------------------------------------

def _inf(a):
    a = np.asarray(a, np.float64)
    a[a <= -1e29] = -np.inf
    return a.astype(np.float32)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_cases(case):
    target = _inf(case["target"])[None]
    draft = _inf(case["draft"])[None]
    K = draft.shape[1]
    res = oracle.verify_sample(target, draft, np.array([case["tokens"]], np.int32),
                               f32([case["T"]]), f32([case["u_accept"]]), f32([case["u_sample"]]))
    assert int(res["n"][0]) == case["expect_n"]
    assert res["out"][0].tolist() == case["expect_out"]
    assert res["p_draft"][0, :K] == pytest.approx(case["expect_p"], abs=1e-7)
    assert res["q_draft"][0, :K] == pytest.approx(case["expect_q"], abs=1e-7)


# --------------------------------------------------------------------------
# greedy verification
# --------------------------------------------------------------------------

def _greedy_invariants(target, tokens, depth, out, n):
    B, K1, V = target.shape
    K = K1 - 1
    vals = synth.as_f64(target)
    for b in range(B):
        d = K if depth is None else int(depth[b])
        g = [int(np.argmax(vals[b, k])) for k in range(d + 1)]
        nb = int(n[b])
        assert 0 <= nb <= d
        assert all(int(tokens[b, k]) == g[k] for k in range(nb))
        if nb < d:
            assert int(tokens[b, nb]) != g[nb]
        assert out[b, :nb].tolist() == tokens[b, :nb].tolist()
        assert int(out[b, nb]) == g[nb]
        assert np.all(out[b, nb + 1:] == -1)


def test_greedy_invariants_random():
    for seed in range(4):
        w = synth.random_case(seed, B=6, K=5, V=700, dtype="bf16", temps=(0.0,), sigma=0.4)
        g = np.random.default_rng(seed)
        depth = g.integers(0, w.K + 1, w.B).astype(np.int32)
        out, n = oracle.verify_greedy(w.target, w.tokens, depth)
        _greedy_invariants(w.target, w.tokens, depth, out, n)
        assert (n > 0).any()


def test_greedy_special_cases():
    g = np.random.default_rng(1)
    B, K, V = 3, 4, 50
    target = g.standard_normal((B, K + 1, V)).astype(np.float32)
    am = np.argmax(target, axis=2).astype(np.int32)
    tokens = am[:, :K].copy()
    out, n = oracle.verify_greedy(target, tokens)
    assert np.all(n == K) and np.array_equal(out, am)          # all accepted + bonus from row K
    tokens[:, 0] = (tokens[:, 0] + 1) % V
    out, n = oracle.verify_greedy(target, tokens)
    assert np.all(n == 0) and np.array_equal(out[:, 0], am[:, 0])
    tokens = am[:, :K].copy()
    tokens[1, 2] = (tokens[1, 2] + 1) % V                       # accept, accept, reject, accept
    depth = np.array([2, 4, 0], np.int32)
    out, n = oracle.verify_greedy(target, tokens, depth)
    assert n.tolist() == [2, 2, 0]
    assert out[0].tolist() == [am[0, 0], am[0, 1], am[0, 2], -1, -1]   # bonus from row d = 2
    assert out[2].tolist() == [am[2, 0], -1, -1, -1, -1]


def test_greedy_bad_inputs():
    g = np.random.default_rng(2)
    B, K, V = 4, 3, 20
    target = g.standard_normal((B, K + 1, V)).astype(np.float32)
    tokens = np.argmax(target, axis=2)[:, :K].astype(np.int32)
    tokens[0, 1] = V            # out of range
    target[1, 2, 5] = np.nan    # NaN inside the window
    target[2, 3, :] = np.nan    # NaN outside the window of depth 2 -> fine
    target[3, 0, :] = -np.inf   # all -inf row
    depth = np.array([3, 3, 2, 3], np.int32)
    out, n = oracle.verify_greedy(target, tokens, depth)
    assert n.tolist() == [-1, -1, 2, -1]
    t2 = target.copy()
    t2[2, 1, 7] = np.inf        # +inf inside the window
    assert oracle.verify_greedy(t2, tokens, depth)[1][2] == -1
    assert np.all(out[[0, 1, 3]] == -1)
    out, n = oracle.verify_greedy(target, tokens, np.array([4, -1, 2, 3], np.int32))
    assert n[0] == -1 and n[1] == -1


# --------------------------------------------------------------------------
# sampled verification: acceptance, losslessness, planted rates
# --------------------------------------------------------------------------

def _tile_case(z_rows, y_rows):
    return np.asarray(z_rows, np.float32), np.asarray(y_rows, np.float32)


def test_acceptance_probability_equals_sum_min_exact_enumeration():
    # K = 1: enumerate the drafted token x (weight q(x)) and a stratified grid
    # of u_accept; the acceptance rate must be sum_v min(p_v, q_v).
    g = np.random.default_rng(4)
    V, N, T = 6, 2000, 0.8
    z = (g.standard_normal(V) * 1.5).astype(np.float32)
    y = (z + g.standard_normal(V)).astype(np.float32)
    p = torch_softmax64(z.astype(np.float64), T)
    q = torch_softmax64(y.astype(np.float64), T)
    B = V * N
    target = np.broadcast_to(np.stack([z, z])[None], (B, 2, V)).copy()
    draft = np.broadcast_to(y[None, None], (B, 1, V)).copy()
    tokens = np.repeat(np.arange(V, dtype=np.int32), N)[:, None]
    ua = np.tile(((np.arange(N) + 0.5) / N).astype(np.float32), V)[:, None]
    res = oracle.verify_sample(target, draft, tokens, np.full(B, T, np.float32), ua,
                               np.zeros(B, np.float32))
    acc = (res["n"] == 1).reshape(V, N).mean(axis=1)
    assert float(np.dot(q, acc)) == pytest.approx(float(np.minimum(p, q).sum()), abs=2.0 / N)


def _lossless_enumeration(z, y, T, N1, N2):
    V = z.shape[0]
    q = torch_softmax64(y.astype(np.float64), T)
    xs, i, j = np.meshgrid(np.arange(V), np.arange(N1), np.arange(N2), indexing="ij")
    B = xs.size
    target = np.broadcast_to(np.stack([z, z])[None], (B, 2, V)).copy()
    draft = np.broadcast_to(y[None, None], (B, 1, V)).copy()
    ua = ((i.ravel() + 0.5) / N1).astype(np.float32)[:, None]
    us = ((j.ravel() + 0.5) / N2).astype(np.float32)
    res = oracle.verify_sample(target, draft, xs.ravel().astype(np.int32)[:, None],
                               np.full(B, T, np.float32), ua, us)
    first = res["out"][:, 0]
    w = np.repeat(q, N1 * N2) / (N1 * N2)
    return np.bincount(first, weights=w, minlength=V)


@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_lossless_exact_enumeration(T):
    # The first emitted token of a K=1 verification, averaged over x ~ q and
    # stratified (u_accept, u_sample) grids, is distributed as p (to O(1/N)).
    g = np.random.default_rng(int(T * 10))
    V = 5
    z = (g.standard_normal(V) * 1.5).astype(np.float32)
    y = (z + g.standard_normal(V) * 1.2).astype(np.float32)
    dist = _lossless_enumeration(z, y, T, 300, 300)
    p = torch_softmax64(z.astype(np.float64), T)
    assert np.max(np.abs(dist - p)) < 4.0 / 300


def test_lossless_with_disjoint_support():
    # draft and target share no token with positive mass except one
    z = _inf([0.0, 0.0, -1e30, -1e30, 1.0])
    y = _inf([-1e30, 0.0, 0.0, 2.0, -1e30])
    dist = _lossless_enumeration(z, y, 1.0, 200, 200)
    p = torch_softmax64(synth.as_f64(z), 1.0)
    assert np.max(np.abs(dist - p)) < 4.0 / 200
    assert dist[2] == 0 and dist[3] == 0


def test_bonus_draw_is_target_row_d_distribution():
    # draft == target at row 0 -> always accepted; bonus comes from row d=1
    g = np.random.default_rng(6)
    V, N = 7, 4000
    z0 = g.standard_normal(V).astype(np.float32)
    z1 = (g.standard_normal(V) * 2).astype(np.float32)
    z2 = (g.standard_normal(V) * 2).astype(np.float32)
    target = np.broadcast_to(np.stack([z0, z1, z2])[None], (N, 3, V)).copy()
    draft = np.broadcast_to(np.stack([z0, z0])[None], (N, 2, V)).copy()
    tokens = np.zeros((N, 2), np.int32)
    us = ((np.arange(N) + 0.5) / N).astype(np.float32)
    res = oracle.verify_sample(target, draft, tokens, np.ones(N, np.float32),
                               np.zeros((N, 2), np.float32), us, depth=np.ones(N, np.int32))
    assert np.all(res["n"] == 1)
    dist = np.bincount(res["out"][:, 1], minlength=V) / N
    assert np.max(np.abs(dist - torch_softmax64(z1.astype(np.float64), 1.0))) < 2.0 / N
    assert np.all(res["out"][:, 2] == -1)


def test_planted_alpha_mean_accepted_length():
    alphas = [0.81, 0.66, 0.52]
    B = 30000
    w = synth.planted_alpha(0, B, alphas, V=12)
    res = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept, w.u_sample)
    n = res["n"]
    expect = sum(np.prod(alphas[:k + 1]) for k in range(len(alphas)))
    se = n.std() / math.sqrt(B)
    assert abs(n.mean() - expect) < 5 * se
    for k, a in enumerate(alphas):       # per-position conditional acceptance
        reached = n >= k
        rate = np.mean(n[reached] > k)
        assert abs(rate - a) < 5 * math.sqrt(a * (1 - a) / reached.sum())
    # accepted-draft probabilities are exactly the planted ones
    m = res["ratio"] < 1
    assert np.all(res["ratio"][m] == 0) and np.all(w.tokens[m] == 11)


def test_lossless_mc_three_positions_chi_square():
    # Fixed-seed Monte Carlo over K = 3 with a small vocabulary: the token
    # emitted at every position, given that it is emitted, follows the
    # target row of that position.
    from scipy.stats import chisquare
    g = np.random.default_rng(12)
    V, K, B, T = 5, 3, 60000, 1.0
    zrows = (g.standard_normal((K + 1, V)) * 1.3).astype(np.float32)
    yrows = (zrows[:K] + g.standard_normal((K, V)) * 0.9).astype(np.float32)
    target = np.broadcast_to(zrows[None], (B, K + 1, V)).copy()
    draft = np.broadcast_to(yrows[None], (B, K, V)).copy()
    tokens = np.empty((B, K), np.int32)
    for k in range(K):
        gum = -np.log(-np.log(g.random((B, V))))
        tokens[:, k] = np.argmax(yrows[k].astype(np.float64)[None] / T + gum, axis=1)
    ua = g.random((B, K), dtype=np.float32)
    us = g.random(B, dtype=np.float32)
    res = oracle.verify_sample(target, draft, tokens, np.full(B, T, np.float32), ua, us)
    n, out = res["n"], res["out"]
    for k in range(K + 1):
        emitted = out[n >= k, k]
        obs = np.bincount(emitted, minlength=V)
        exp = torch_softmax64(zrows[k].astype(np.float64), T) * emitted.size
        assert chisquare(obs, exp).pvalue > 1e-3


def test_temperature_applies_to_both_rows():
    # p_draft / q_draft are softmax(z/T)[x] and softmax(y/T)[x] (torch float64)
    w = synth.random_case(3, B=5, K=3, V=300, dtype="f32", temps=(0.5, 1.3), sigma=1.0)
    res = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept, w.u_sample)
    for b in range(w.B):
        T = float(w.temperature[b])
        for k in range(w.K):
            x = int(w.tokens[b, k])
            assert res["p_draft"][b, k] == np.float32(torch_softmax64(synth.as_f64(w.target[b, k]), T)[x])
            assert res["q_draft"][b, k] == np.float32(torch_softmax64(synth.as_f64(w.draft[b, k]), T)[x])


def test_first_rejection_not_total_accepts():
    # accept, reject, accept: n must be 1 even though two tokens pass the test
    V = 4
    z = _inf([[0, 0, 0, 0]] * 4)
    y = _inf([[0, -1e30, -1e30, 0]] * 3)     # ratio for x=0 is 1/2 at every position
    res = oracle.verify_sample(z[None], y[None], np.zeros((1, 3), np.int32), f32([1.0]),
                               f32([[0.1, 0.9, 0.1]]), f32([0.0]))
    assert int(res["n"][0]) == 1
    assert res["out"][0].tolist() == [0, 1, -1, -1]


def test_sample_bad_inputs_and_window():
    w = synth.random_case(1, B=6, K=3, V=64, dtype="f32", temps=(1.0,))
    t, d = w.target.copy(), w.draft.copy()
    tok, ua, us, T = w.tokens.copy(), w.u_accept.copy(), w.u_sample.copy(), w.temperature.copy()
    depth = np.array([3, 3, 3, 1, 3, 3], np.int32)
    tok[0, 2] = -1              # out of range
    ua[1, 0] = 1.0              # uniform outside [0, 1)
    T[2] = -0.5                 # negative temperature
    d[3, 2, :] = np.nan         # NaN outside the window of depth 1 -> fine
    d[4, 1, 3] = np.nan         # NaN in a draft row inside the window
    T[5] = np.nan
    res = oracle.verify_sample(t, d, tok, T, ua, us, depth)
    assert res["n"].tolist()[:3] == [-1, -1, -1]
    assert res["n"][3] >= 0 and res["n"][4] == -1 and res["n"][5] == -1
    T2 = w.temperature.copy()
    # +-inf and -0.5 are bad; every finite T > 0 is a temperature, fp32
    # denormals and the largest fp32 value included
    T2[:6] = [np.inf, -np.inf, -0.5, 1e-7, 2e6, np.float32(1e-45)]
    res2 = oracle.verify_sample(w.target, w.draft, w.tokens, T2, w.u_accept, w.u_sample)
    assert res2["n"].tolist()[:3] == [-1, -1, -1] and np.all(res2["n"][3:6] >= 0)
    T3 = np.full_like(T2, np.float32(3.4028235e38))
    assert np.all(oracle.verify_sample(w.target, w.draft, w.tokens, T3, w.u_accept, w.u_sample)["n"] >= 0)
    assert np.all(res["out"][[0, 1, 2, 4, 5]] == -1)
    assert np.all(res["p_draft"][3, 1:] == 0)


def test_zero_temperature_request_uses_greedy_rule():
    w = synth.random_case(7, B=8, K=4, V=200, dtype="bf16", temps=(0.0,), sigma=0.3)
    res = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept, w.u_sample)
    out, n = oracle.verify_greedy(w.target, w.tokens)
    assert np.array_equal(res["out"], out) and np.array_equal(res["n"], n)
    assert np.all(res["p_draft"] == 0)


# --------------------------------------------------------------------------
# early-exit verification: positions in order, nothing read after the stop
# --------------------------------------------------------------------------

def _poison_after_stop(w, depth, n):
    """NaN rows, out-of-range tokens and invalid uniforms at every position
    after each request's stopping position (what an early-exit reading never
    reads)."""
    t, tok = w.target.copy(), w.tokens.copy()
    d_ = None if w.draft is None else w.draft.copy()
    ua = None if w.u_accept is None else w.u_accept.copy()
    nan = synth.to_bf16_bits(np.array([np.nan], np.float32))[0] if t.dtype == np.uint16 else np.nan
    for b in range(w.B):
        nb, db = int(n[b]), int(depth[b])
        if 0 <= nb < db:
            t[b, nb + 1:, :] = nan
            tok[b, nb + 1:] = -3
            if d_ is not None:
                d_[b, nb + 1:, :] = nan
                ua[b, nb + 1:] = 2.0
    return t, d_, tok, ua


def test_early_exit_greedy_invariants_and_nothing_read_after_stop():
    for seed in range(3):
        w = synth.random_case(seed, B=7, K=5, V=300, dtype="f32", temps=(0.0,), sigma=0.4)
        depth = np.random.default_rng(seed).integers(0, w.K + 1, w.B).astype(np.int32)
        res = oracle.verify_early_exit(w.target, w.tokens, depth=depth)
        _greedy_invariants(w.target, w.tokens, depth, res["out"], res["n"])
        stopped = (res["n"] < depth)
        assert stopped.any()
        t2, _, tok2, _ = _poison_after_stop(w, depth, res["n"])
        res2 = oracle.verify_early_exit(t2, tok2, depth=depth)
        assert np.array_equal(res2["out"], res["out"]) and np.array_equal(res2["n"], res["n"])
        # the one-pass rule reads the whole window, so the same data is bad there
        _, n1 = oracle.verify_greedy(t2, tok2, depth)
        assert np.all(n1[stopped] == -1) and np.array_equal(n1[~stopped], res["n"][~stopped])


def test_early_exit_greedy_bad_data_before_stop_and_bonus_row():
    g = np.random.default_rng(5)
    B, K, V = 4, 4, 30
    target = g.standard_normal((B, K + 1, V)).astype(np.float32)
    am = np.argmax(target, axis=2).astype(np.int32)
    tokens = am[:, :K].copy()
    tokens[:, 2] = (am[:, 2] + 1) % V          # every request rejects at position 2
    target[0, 1, 3] = np.nan                    # before the stop: bad
    target[1, 2, :] = -np.inf                   # at the stop: bad
    tokens[2, 3] = V + 7                        # after the stop: never read
    tokens[3, 2] = am[3, 2]                     # request 3 accepts everything ...
    target[3, K, 0] = np.inf                    # ... and its bonus row is bad
    res = oracle.verify_early_exit(target, tokens)
    assert res["n"].tolist() == [-1, -1, 2, -1]
    assert res["out"][2].tolist() == [am[2, 0], am[2, 1], am[2, 2], -1, -1]
    assert np.all(res["out"][[0, 1, 3]] == -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_exit_sampled_equals_one_pass_on_clean_data(dtype):
    for seed in range(3):
        w = synth.random_case(seed, B=9, K=6, V=64, dtype=dtype, temps=(0.0, 0.7, 1.0), sigma=0.8)
        depth = np.random.default_rng(10 + seed).integers(0, w.K + 1, w.B).astype(np.int32)
        ee = oracle.verify_early_exit(w.target, w.tokens, w.draft, w.temperature, w.u_accept,
                                      w.u_sample, depth)
        full = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept,
                                    w.u_sample, depth)
        assert np.array_equal(ee["out"], full["out"]) and np.array_equal(ee["n"], full["n"])
        for b in range(w.B):
            m = min(int(ee["n"][b]), int(depth[b]) - 1)   # last position read
            for key in ("p_draft", "q_draft"):
                assert np.array_equal(ee[key][b, :m + 1], full[key][b, :m + 1])
                assert np.all(ee[key][b, m + 1:] == 0)
        t2, d2, tok2, ua2 = _poison_after_stop(w, depth, ee["n"])
        ee2 = oracle.verify_early_exit(t2, tok2, d2, w.temperature, ua2, w.u_sample, depth)
        for key in ("out", "n", "p_draft", "q_draft"):
            assert np.array_equal(ee2[key], ee[key])


def test_early_exit_sampled_hand_case():
    # target uniform over 4 tokens, draft uniform over tokens {0, 3}: the
    # ratio at x = 0 is (1/4)/(1/2) = 1/2 at every position.  u = 0.1 accepts,
    # 0.9 rejects; position 2 comes after the stop and is not read, so its
    # invalid uniform and NaN rows do not matter and its p/q stay 0.
    z = _inf([[0, 0, 0, 0]] * 4)
    y = _inf([[0, -1e30, -1e30, 0]] * 3)
    z[2, 1] = np.nan
    y[2, 2] = np.nan
    res = oracle.verify_early_exit(z[None], np.zeros((1, 3), np.int32), y[None], f32([1.0]),
                                   f32([[0.1, 0.9, 7.0]]), f32([0.0]))
    assert int(res["n"][0]) == 1
    # residual at position 1: max(0, 1/4 - q) is 1/4 on tokens 1 and 2; u = 0 takes token 1
    assert res["out"][0].tolist() == [0, 1, -1, -1]
    assert res["p_draft"][0].tolist() == [0.25, 0.25, 0.0]
    assert res["q_draft"][0].tolist() == [0.5, 0.5, 0.0]
    # the one-pass rule reads position 2 and reports the request as bad
    full = oracle.verify_sample(z[None], y[None], np.zeros((1, 3), np.int32), f32([1.0]),
                                f32([[0.1, 0.9, 7.0]]), f32([0.0]))
    assert int(full["n"][0]) == -1
    # the accept test is strict: u equal to the ratio rejects
    tie = oracle.verify_early_exit(z[None], np.zeros((1, 3), np.int32), y[None], f32([1.0]),
                                   f32([[0.5, 0.1, 0.1]]), f32([0.0]))
    assert int(tie["n"][0]) == 0
    # a bad uniform before the stop, and a bad draw uniform, are bad data
    assert int(oracle.verify_early_exit(z[None], np.zeros((1, 3), np.int32), y[None], f32([1.0]),
                                        f32([[1.0, 0.9, 0.1]]), f32([0.0]))["n"][0]) == -1
    assert int(oracle.verify_early_exit(z[None], np.zeros((1, 3), np.int32), y[None], f32([1.0]),
                                        f32([[0.1, 0.9, 0.1]]), f32([1.0]))["n"][0]) == -1


# --------------------------------------------------------------------------
# draft confidence
# --------------------------------------------------------------------------

def test_draft_confidence_is_max_softmax():
    w = synth.random_case(2, B=3, K=4, V=900, dtype="bf16")
    kb = np.array([4, 2, 0], np.int32)
    conf = oracle.draft_confidence(w.draft, kb)
    for b in range(w.B):
        for k in range(w.K):
            if k >= kb[b]:
                assert conf[b, k] == 0
            else:
                ref = torch_softmax64(synth.as_f64(w.draft[b, k]), 1.0).max()
                assert conf[b, k] == pytest.approx(ref, rel=1.2e-7)


# --------------------------------------------------------------------------
# D-cut allocation
# --------------------------------------------------------------------------

def _prefix_conf(conf, Kb):
    c = np.zeros_like(conf)
    for b in range(conf.shape[0]):
        if Kb[b] > 0:
            c[b, :Kb[b]] = np.cumprod(np.clip(np.nan_to_num(conf[b, :Kb[b]], nan=0.0), 0, 1),
                                      dtype=np.float32)
    return c


def test_dcut_bruteforce_optimum():
    g = np.random.default_rng(21)
    for trial in range(150):
        B = int(g.integers(1, 6))
        K = int(g.integers(1, 5))
        Kb = g.integers(1, K + 1, B).astype(np.int32)
        conf = g.uniform(0.05, 1.0, (B, K)).astype(np.float32)
        if trial % 3 == 0:
            conf = np.round(conf * 4) / 4            # force ties
            conf[conf == 0] = 0.25
        budget = int(g.integers(B, int(Kb.sum()) + 3))
        d = oracle.dcut_allocate(conf, budget, Kb)
        c = _prefix_conf(conf, Kb).astype(np.float64)
        total = min(budget, int(Kb.sum()))
        assert int(d.sum()) == total
        assert np.all((d >= 1) & (d <= Kb))
        best, best_vecs = -1.0, []
        for vec in itertools.product(*[range(1, int(k) + 1) for k in Kb]):
            if sum(vec) != total:
                continue
            val = sum(c[b, :vec[b]].sum() for b in range(B))
            if val > best + 1e-12:
                best, best_vecs = val, [vec]
            elif abs(val - best) <= 1e-12:
                best_vecs.append(vec)
        got = sum(c[b, :d[b]].sum() for b in range(B))
        assert got == pytest.approx(best, abs=1e-12)
        if len(best_vecs) == 1:
            assert tuple(d.tolist()) == best_vecs[0]


def test_dcut_special_cases():
    g = np.random.default_rng(22)
    B, K = 6, 5
    conf = g.uniform(0.1, 1, (B, K)).astype(np.float32)
    assert np.all(oracle.dcut_allocate(conf, B) == 1)
    assert np.all(oracle.dcut_allocate(conf, B * K) == K)
    assert np.all(oracle.dcut_allocate(conf, 10 * B * K) == K)
    eq = np.full((3, 3), 0.5, np.float32)         # equal prefixes: lowest flat index first
    assert oracle.dcut_allocate(eq, 5).tolist() == [2, 2, 1]
    assert oracle.dcut_allocate(eq, 7).tolist() == [3, 2, 2]
    with pytest.raises(ValueError):
        oracle.dcut_allocate(conf, B - 1)


def test_dcut_float_cumprod_and_sanitising():
    # the ranking key is the float32 running product (numpy float32 cumprod)
    conf = np.array([[0.3, 0.7, 0.9, 0.2], [0.9, 0.9, 0.1, 0.9]], np.float32)
    c = np.cumprod(conf, axis=1, dtype=np.float32)
    entries = sorted(((-c[b, k], b * 4 + k, b) for b in range(2) for k in range(1, 4)))
    for budget in range(2, 9):
        d = [1, 1]
        for e in entries[:budget - 2]:
            d[e[2]] += 1
        assert oracle.dcut_allocate(conf, budget).tolist() == d
    bad = np.array([[np.nan, 0.9], [-1.0, 0.9], [2.0, 0.5]], np.float32)
    # NaN / negative count as 0, values above 1 as 1: only request 2 has a positive prefix
    assert oracle.dcut_allocate(bad, 4).tolist() == [1, 1, 2]
    tiny = np.full((2, 16), 1e-4, np.float32)       # products underflow through denormals to 0
    d = oracle.dcut_allocate(tiny, 20)
    assert d.tolist() == [11, 9] or d.sum() == 20
    c = np.cumprod(tiny[0], dtype=np.float32)
    assert c[-1] == 0 and (c > 0).sum() > 9         # denormals are kept, not flushed


def test_dcut_invalid_max_depth():
    conf = np.full((3, 4), 0.9, np.float32)
    d = oracle.dcut_allocate(conf, 8, np.array([4, 5, 0], np.int32))
    assert d.tolist() == [4, -1, 0]


# --------------------------------------------------------------------------
# metric definition printed by the pages
# --------------------------------------------------------------------------

def test_metric_definition_tau_counts_bonus():
    m = json.load(open(os.path.join(GOLDEN, "metric_definition.json")))
    K = m["K"]
    for pair in m["pairs"]:
        assert abs((1 + K * pair["rate"]) - pair["tau"]) <= m["print_rounding"]["tau"] + K * m["print_rounding"]["rate"]
        assert abs(pair["rate"] * K - pair["tau"]) > 0.3      # tau does not exclude the bonus


# ------------------------------------------------- acceptance statistics ----

def test_accept_stats_hand_case():
    # n = (0, 2, 3, bad, 1) with windows (3, 3, 3, 3, 1), K = 3, worked by hand:
    # position 0 is tested by every valid request, accepted by all but the first;
    # position 1 by the two that got past 0 inside a 3-wide window; and so on.
    n = np.array([0, 2, 3, -1, 1], np.int32)
    d = np.array([3, 3, 3, 3, 1], np.int32)
    c = oracle.accept_stats(n, 3, d)
    assert c.tolist() == [4, 2, 2, 3, 2, 1, 4, 1, 6, 10]


def test_accept_stats_invariants_and_accumulation():
    g = np.random.default_rng(5)
    K, B = 7, 500
    d = g.integers(0, K + 1, B).astype(np.int32)
    n = np.minimum(g.integers(0, K + 1, B), d).astype(np.int32)
    n[g.random(B) < 0.05] = -1
    c = oracle.accept_stats(n, K, d)
    ok = n >= 0
    reached, accepted = c[:K].astype(np.int64), c[K:2 * K].astype(np.int64)
    # every accepted draft is counted once at its position
    assert accepted.sum() == np.minimum(n[ok], d[ok]).sum()
    # a tested position that was not accepted is exactly one rejection
    rej = np.bincount(n[ok & (n < d)], minlength=K)[:K]
    assert np.array_equal(reached - accepted, rej)
    assert c[2 * K] == ok.sum() and c[2 * K + 1] == (~ok).sum()
    assert c[2 * K + 2] == n[ok].sum() and c[2 * K + 3] == n[ok].sum() + ok.sum()
    # the counters add across calls
    c2 = oracle.accept_stats(n, K, d, c.copy())
    assert np.array_equal(c2, 2 * c)
    # positions outside the window are never counted; NULL depth means K
    c3 = oracle.accept_stats(np.array([5], np.int32), 3, np.array([9], np.int32))
    assert c3[:3].tolist() == [1, 1, 1] and c3[3:6].tolist() == [1, 1, 1]
    assert np.array_equal(oracle.accept_stats(n, K), oracle.accept_stats(n, K, np.full(B, K, np.int32)))


# ------------------------------------------------------- cost-aware D-cut ----

def test_dcut_cost_interpolation_hand_values():
    # the pages' latency table: 1 -> 1.0, 2 -> 1.2, 4 -> 1.5, 8 -> 2.0, 16 -> 3.0
    want = {0.5: 1.0, 1: 1.0, 2: 1.2, 3: 1.35, 4: 1.5, 5: 1.625, 6: 1.75, 8: 2.0, 12: 2.5, 16: 3.0, 40: 3.0}
    for d, c in want.items():
        assert abs(oracle.dcut_cost(d) - c) < 1e-15, (d, oracle.dcut_cost(d), c)


def test_dcut_cost_table_points_and_segments():
    # at a table depth the cost is that point's own value, bit for bit; between two
    # points it lies on the chord (checked against a fraction computed separately)
    from fractions import Fraction
    g = np.random.default_rng(17)
    for trial in range(20):
        n = int(g.integers(1, 12))
        t = np.cumsum(g.integers(1, 5, n)).astype(np.float64)
        c = np.cumsum(g.uniform(0.05, 2.0, n))
        table = tuple(zip(t.tolist(), c.tolist()))
        for ti, ci in table:
            assert oracle.dcut_cost(ti, table) == ci
        assert oracle.dcut_cost(t[0] - 0.5, table) == c[0] and oracle.dcut_cost(t[-1] + 3, table) == c[-1]
        for i in range(n - 1):
            d = float(t[i] + 0.5 * (t[i + 1] - t[i]))
            exact = Fraction(c[i]) + (Fraction(d) - Fraction(t[i])) / (Fraction(t[i + 1]) - Fraction(t[i])) \
                * (Fraction(c[i + 1]) - Fraction(c[i]))
            assert abs(oracle.dcut_cost(d, table) - float(exact)) <= 4e-16 * float(exact)


def test_dcut_cost_choices_closed_forms():
    # confidence 1 everywhere: benefit d / cost(d) grows with d on this table, so the
    # whole window is chosen (16 / 3.0 at K_b = 16; 5 / 1.625 beats 4 / 1.5 at K_b = 5)
    conf = np.ones((2, 16), np.float32)
    assert oracle.dcut_allocate_cost(conf, 100.0, np.array([16, 5], np.int32)).tolist() == [16, 5]
    # a zero after the first position: every longer prefix has benefit 0, so depth 1
    conf = np.zeros((1, 8), np.float32)
    conf[0, 0] = 0.9
    assert oracle.dcut_allocate_cost(conf, 100.0).tolist() == [1]
    # NaN, negatives and values above 1 are read as 0, 0 and 1
    conf = np.array([[np.nan, 1.0], [2.0, -1.0]], np.float32)
    assert oracle.dcut_allocate_cost(conf, 100.0).tolist() == [1, 1]
    # invalid windows and empty ones
    conf = np.ones((3, 4), np.float32)
    assert oracle.dcut_allocate_cost(conf, 100.0, np.array([0, 5, -1], np.int32)).tolist() == [0, -1, -1]


def test_dcut_cost_budget_fill_order_and_skip():
    # equal benefits: admitted in request order until the budget runs out (cost 3.0 each)
    conf = np.ones((4, 16), np.float32)
    assert oracle.dcut_allocate_cost(conf, 9.0).tolist() == [16, 16, 16, 0]
    assert oracle.dcut_allocate_cost(conf, 8.999).tolist() == [16, 16, 0, 0]
    # a candidate that does not fit is skipped and a later, cheaper one still fits:
    # request 0 wants depth 16 (benefit 5.33, cost 3.0); request 1 stops at depth 1
    # (benefit 0.5, cost 1.0); with 2.5 of budget only request 1 is admitted
    conf = np.ones((2, 16), np.float32)
    conf[1, :] = 0.0
    conf[1, 0] = 0.5
    assert oracle.dcut_allocate_cost(conf, 2.5).tolist() == [0, 1]
    assert oracle.dcut_allocate_cost(conf, 4.0).tolist() == [16, 1]
    # with room for one of the two, the higher value (request 0) is offered first
    assert oracle.dcut_allocate_cost(conf, 3.0).tolist() == [16, 0]
    # invariant on random inputs: admitted cost within budget, and every candidate left
    # out met a budget too small for it
    g = np.random.default_rng(11)
    conf = g.uniform(0.3, 1.0, (40, 16)).astype(np.float32)
    dep = oracle.dcut_allocate_cost(conf, 30.0)
    costs = [oracle.dcut_cost(d) for d in dep if d > 0]
    assert sum(costs) <= 30.0 and min(dep) >= 0


# --------------------------------------------------------------------------
# temperature range and large logits: the definition has no bound on T > 0
# and is invariant to a constant shift of a row
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1e-30, 1e-40, 1e-45])
def test_sample_vanishing_temperature_is_greedy(T):
    # softmax(z / T) tends to the indicator of the argmax as T falls to 0, so
    # with distinct row maxima the sampled rule accepts exactly the argmax
    # drafts, and the correction or bonus token is the target argmax: the
    # greedy continuation.  Draft tokens are the draft argmax (q(x) = 1).
    w = synth.random_case(21, B=16, K=4, V=3000, dtype="f32", temps=(1.0,), sigma=2.0)
    vals = synth.as_f64(w.target)
    srt = np.sort(vals, axis=2)
    assert np.all(srt[..., -1] > srt[..., -2])
    tok = np.argmax(synth.as_f64(w.draft), axis=2).astype(np.int32)
    Tz = np.full(w.B, np.float32(T), np.float32)
    res = oracle.verify_sample(w.target, w.draft, tok, Tz, w.u_accept, w.u_sample)
    out, n = oracle.verify_greedy(w.target, tok)
    assert np.array_equal(res["out"], out) and np.array_equal(res["n"], n)
    assert set(np.unique(res["p_draft"][res["p_draft"] != 0]).tolist()) <= {1.0}
    assert 0 < n.mean() < w.K


@pytest.mark.parametrize("shift", [2.0 ** 20, -(2.0 ** 20)])
def test_sample_shift_invariance(shift):
    # logits on a grid of 1/8 with |z| < 64 stay exact in fp32 after adding
    # +-2^20, so the shifted rows hold the same distribution exactly; softmax
    # is invariant to a constant added to a row, and an oracle that
    # exponentiates without first subtracting the row maximum would overflow
    g = np.random.default_rng(5)
    B, K, V = 12, 3, 2000
    z = np.clip(np.round(g.standard_normal((B, K + 1, V)) * 24) / 8, -63, 63).astype(np.float32)
    y = np.clip(np.round((z[:, :K] + g.standard_normal((B, K, V)) * 0.4) * 8) / 8, -63, 63).astype(np.float32)
    tok = np.argmax(y.astype(np.float64) + g.gumbel(size=y.shape), axis=2).astype(np.int32)
    T = g.choice(np.array([1.0, 0.7, 2.0], np.float32), B)
    ua, us = g.random((B, K), dtype=np.float32), g.random(B, dtype=np.float32)
    base = oracle.verify_sample(z, y, tok, T, ua, us)
    zs, ys = (z + np.float32(shift)).astype(np.float32), (y + np.float32(shift)).astype(np.float32)
    assert np.array_equal(zs.astype(np.float64) - shift, z.astype(np.float64))
    moved = oracle.verify_sample(zs, ys, tok, T, ua, us)
    for key in ("out", "n", "p_draft", "q_draft"):
        assert np.array_equal(base[key], moved[key]), key
    assert np.all(base["n"] >= 0)
