"""Parity at the vocabulary limit (V = 2,000,000, the largest V the library
accepts; 977 sampler units and the most row-pass chunks a row can have), for
the one-pass and the early-exit calls, bf16 with V a multiple of the vector
width and fp32 with a ragged tail."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import Tally, compare_greedy, compare_sample, dev, host, run_greedy, run_sample

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


@pytest.mark.parametrize("dtype,V", [("bf16", 2_000_000), ("f32", 1_999_999)])
def test_vocabulary_limit(dtype, V):
    import draft_verification_verify_amd as sv
    note(f"vocabulary limit {dtype} V={V}: greedy, sampled and early-exit calls")
    w = synth.random_case(V % 97, B=3, K=2, V=V, dtype=dtype, temps=(0.0, 0.8, 1.0), sigma=0.3)
    depth = np.array([2, 1, 2], np.int32)
    out, n = run_greedy(w, depth)
    assert len(compare_greedy(w, out, n, depth)) == 0
    tal = Tally()
    out, n, p, q = run_sample(w, depth)
    compare_sample(w, out, n, p, q, depth, tal)
    ora = oracle.verify_early_exit(w.target, w.tokens, w.draft, w.temperature, w.u_accept, w.u_sample, depth)
    res = sv.verify_sample_early_exit(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                      dev(w.u_accept), dev(w.u_sample), dev(depth), ends=[1, 2])
    torch.cuda.synchronize()
    eo, en = host(res[0]), host(res[1])
    # clean data: the one-pass oracle's ratios are those of the positions read
    full = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept, w.u_sample, depth)
    compare_sample(w, eo, en, None, None, depth, tal, dict(ora, ratio=full["ratio"]))
    tal.assert_ok(f"{dtype} V={V}")
