"""Determinism across decompositions of the same work, through the C ABI.

SPECVERIFY_CHUNK forces the number of chunks each logit row is split into
by the row-statistics pass (a different assignment of work to waves, a
different order of partial sums and merges).  Greedy outputs and D-cut
depths must be bit-identical across chunk counts and repeated calls;
sampled tokens and accepted counts bit-identical as well (their decisions
sit far from the tolerance bands on these seeds), with p/q and confidence
within rounding of each other and within the stated tolerances of the
oracle."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import compare_greedy, compare_sample, dev, host, run_greedy, run_sample

pytestmark = pytest.mark.gpu

CHUNKS = [None, 1, 2, 7, 64, 256]


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    import draft_verification_verify_amd  # noqa: F401
    yield
    os.environ.pop("SPECVERIFY_CHUNK", None)


def with_chunks(n, fn):
    if n is None:
        os.environ.pop("SPECVERIFY_CHUNK", None)
    else:
        os.environ["SPECVERIFY_CHUNK"] = str(n)
    try:
        return fn()
    finally:
        os.environ.pop("SPECVERIFY_CHUNK", None)


def test_greedy_and_sampled_across_chunk_counts():
    import draft_verification_verify_amd as sv
    wg = synth.dcut_ragged(7, T=0.0, B=16)
    ws = synth.dcut_ragged(7, T=1.0, B=16)
    wm = synth.mixed(1, B=16)
    depth_m = wm.max_depth.copy()
    base = None
    for n in CHUNKS:
        note(f"chunks per row = {n}: greedy, sampled (bf16 V=128000) and mixed fp32 V=152064")
        res = with_chunks(n, lambda: (run_greedy(wg), run_sample(ws), run_sample(wm, depth_m),
                                      host(sv.draft_confidence(dev(ws.draft)))))
        for _ in range(1):   # the same decomposition twice
            again = with_chunks(n, lambda: run_greedy(wg))
            assert all(np.array_equal(a, b) for a, b in zip(res[0], again))
        assert len(compare_greedy(wg, *res[0])) == 0
        compare_sample(ws, *res[1]).assert_ok(f"sampled chunks={n}")
        compare_sample(wm, *res[2], depth_m).assert_ok(f"mixed chunks={n}")
        if base is None:
            base = res
            continue
        assert all(np.array_equal(a, b) for a, b in zip(base[0], res[0])), n
        for i in (1, 2):
            assert np.array_equal(base[i][0], res[i][0]) and np.array_equal(base[i][1], res[i][1]), (n, i)
            assert np.max(np.abs(base[i][2] - res[i][2])) <= 1e-6 and np.max(np.abs(base[i][3] - res[i][3])) <= 1e-6
        assert np.max(np.abs(base[3] - res[3]) / base[3]) < 1e-6


def test_dcut_pipeline_across_chunk_counts():
    import draft_verification_verify_amd as sv
    w = synth.dcut_ragged(2, T=1.0)
    conf_o = oracle.draft_confidence(w.draft)
    want = oracle.dcut_allocate(conf_o, w.budget)
    for n in CHUNKS:
        note(f"dcut_allocate on fixed confidence, chunks per row = {n}")
        got = with_chunks(n, lambda: host(sv.dcut_allocate(dev(conf_o), w.budget)))
        assert np.array_equal(got, want), n
