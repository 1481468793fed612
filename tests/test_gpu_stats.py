"""GPU parity of spec_accept_stats_update (per-position acceptance counters
across calls) against the oracle, through the C ABI, and its planted-rate
check against the closed form."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import dev, host, run_sample

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    import draft_verification_verify_amd  # noqa: F401


@pytest.mark.parametrize("B,K", [(1, 0), (1, 1), (7, 3), (64, 16), (4096, 16), (300, 1024)])
def test_accept_stats_random_bit_exact(B, K):
    note(f"accept stats random B={B} K={K}, three calls accumulated")
    import draft_verification_verify_amd as sv
    g = np.random.default_rng(B * 31 + K)
    counters = None
    expect = np.zeros(2 * K + 4, np.uint64)
    for call in range(3):
        d = g.integers(-1, K + 3, B).astype(np.int32)          # windows past K and negative ones too
        n = g.integers(-1, K + 2, B).astype(np.int32)          # n past the window, and bad requests
        use_depth = call != 1
        counters = sv.accept_stats_update(dev(n), K, dev(d) if use_depth else None, counters)
        expect = oracle.accept_stats(n, K, d if use_depth else None, expect)
    torch.cuda.synchronize()
    assert np.array_equal(host(counters).astype(np.uint64), expect)


def test_accept_stats_planted_alpha():
    note("accept stats on planted acceptance rates: alpha_hat_k ~ alpha_k, tau = mean + 1")
    import draft_verification_verify_amd as sv
    alphas = [0.81, 0.66, 0.52]
    B = 4000
    w = synth.planted_alpha(2, B, alphas, V=12)
    out, n, p, q = run_sample(w)
    c = sv.accept_stats_update(dev(n), len(alphas))
    torch.cuda.synchronize()
    assert np.array_equal(host(c).astype(np.uint64), oracle.accept_stats(n, len(alphas)))
    s = sv.accept_stats_summary(c, len(alphas))
    assert s["requests"] == B and s["bad"] == 0
    for k, a in enumerate(alphas):
        r = s["reached"][k]
        assert abs(s["alpha"][k] - a) < 5 * np.sqrt(a * (1 - a) / r), (k, s["alpha"][k], a)
    assert abs(s["mean_accepted"] - n.mean()) < 1e-12
    assert abs(s["tau"] - (n.mean() + 1)) < 1e-12


def test_accept_stats_after_ragged_verify():
    note("accept stats of a ragged sampled verify (D-cut depths) equal the oracle's on the same outputs")
    import draft_verification_verify_amd as sv
    w = synth.random_case(91, B=48, K=16, V=5000, dtype="bf16", temps=(0.0, 0.7, 1.0))
    depth = np.random.default_rng(3).integers(0, 17, 48).astype(np.int32)
    out, n, p, q = run_sample(w, depth)
    c = sv.accept_stats_update(dev(n), 16, dev(depth))
    torch.cuda.synchronize()
    assert np.array_equal(host(c).astype(np.uint64), oracle.accept_stats(n, 16, depth))
