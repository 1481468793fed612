"""GPU parity of the packed (CSR) layout calls, spec_verify_greedy_packed and
spec_verify_sample_packed, through the C ABI.

Request b's drafted positions are offsets[b] .. offsets[b+1]-1 of flat
arrays; its d_b + 1 target rows and output slots start at offsets[b] + b.
The oracle verifies the padded workload with depth d_b; the packed inputs
are a copy of exactly the rows and slots that depth reads (everything else
in the packed arrays is NaN or invalid, so a stray read shows up), and the
packed outputs are compared, after unpacking, by the padded rules.  Where
the rows keep their 16-byte alignment the packed call must also match the
padded GPU call bit for bit (same plan, same chunking, same kernels).
Cases: the D-cut batch at budget 384 (B=64, K=16, V=128000 bf16), the
mixed fp32 batch at budget 512 (V=152064, per-request K_b and T), greedy,
shapes with V not a multiple of the vector width, offsets not starting at
0, unused slack, depth 0, K_max above every depth, and bad offsets."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (Packed, compare_greedy, compare_sample, run_greedy, run_greedy_packed, run_sample,
                    run_sample_packed)

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


def sample_packed_check(w, depth, K_max, start=0, slack=0, padded_identical=True, label=""):
    pk = Packed(w, depth, start=start, slack=slack)
    out, n, p, q = run_sample_packed(pk, w, K_max)
    out_pad, p_pad, q_pad, unowned = pk.unpack(w, out, p, q)
    assert np.all(out[unowned] == -99), f"{label}: a slot no request owns was written"
    tal = compare_sample(w, out_pad, n, p_pad, q_pad, depth)
    tal.assert_ok(label)
    if padded_identical:
        o2, n2, p2, q2 = run_sample(w, depth)
        assert np.array_equal(o2, out_pad) and np.array_equal(n2, n), f"{label}: packed != padded"
        assert np.array_equal(p2, p_pad) and np.array_equal(q2, q_pad), f"{label}: packed p/q != padded"
    return n


def test_packed_sample_dcut_budget384():
    note("packed sample: D-cut batch B=64 K=16 V=128000 bf16, budget 384 (depths from dcut_allocate)")
    w = synth.dcut_ragged(0, T=1.0)
    depth = oracle.dcut_allocate(oracle.draft_confidence(w.draft), w.budget)
    assert int(depth.sum()) == 384
    n = sample_packed_check(w, depth, w.K, label="dcut 384")
    assert np.all(n >= 0)


def test_packed_sample_mixed_budget512():
    note("packed sample: mixed fp32 batch B=64 V=152064, per-request K_b and T, budget 512")
    w = synth.mixed(0)
    depth = oracle.dcut_allocate(oracle.draft_confidence(w.draft, w.max_depth), w.budget, w.max_depth)
    n = sample_packed_check(w, depth, w.K, start=5, slack=3, label="mixed 512")
    assert np.all(n >= 0)


def test_packed_greedy_dcut_budget384():
    note("packed greedy: D-cut batch at T=0, budget 384")
    w = synth.dcut_ragged(1, T=0.0)
    depth = oracle.dcut_allocate(oracle.draft_confidence(w.draft), w.budget)
    pk = Packed(w, depth, start=2, slack=1)
    out, n = run_greedy_packed(pk, w.K)
    out_pad, _, _, unowned = pk.unpack(w, out)
    assert np.all(out[unowned] == -99)
    assert len(compare_greedy(w, out_pad, n, depth)) == 0
    o2, n2 = run_greedy(w, depth)
    assert np.array_equal(o2, out_pad) and np.array_equal(n2, n)


@pytest.mark.parametrize("dtype,V,K", [("bf16", 1003, 5), ("f32", 777, 7), ("bf16", 4096, 16), ("f32", 33, 3)])
def test_packed_fuzz_shapes(dtype, V, K):
    note(f"packed fuzz {dtype} V={V} K={K}: random depths (0 included), offset start, slack, K_max > depths")
    g = np.random.default_rng(1000 + V)
    for seed in range(3):
        B = int(g.integers(1, 24))
        w = synth.random_case(seed, B=B, K=K, V=V, dtype=dtype, temps=(0.0, 0.7, 1.0))
        depth = g.integers(0, K + 1, B).astype(np.int32)
        aligned = (V * (2 if dtype == "bf16" else 4)) % 16 == 0
        sample_packed_check(w, depth, K + int(g.integers(0, 3)), start=int(g.integers(0, 4)),
                            slack=int(g.integers(0, 3)), padded_identical=aligned, label=f"fuzz seed {seed}")
        pk = Packed(w, depth, start=1)
        out, n = run_greedy_packed(pk, K)
        out_pad, _, _, unowned = pk.unpack(w, out)
        assert np.all(out[unowned] == -99)
        assert len(compare_greedy(w, out_pad, n, depth)) == 0


def test_packed_no_drafted_positions():
    note("packed: every depth 0 (no draft arrays; bonus tokens only)")
    w = synth.random_case(4, B=5, K=3, V=1000, dtype="f32", temps=(0.0, 1.0))
    depth = np.zeros(5, np.int32)
    pk = Packed(w, depth)
    assert pk.N == 0
    out, n, p, q = run_sample_packed(pk, w, 3)
    out_pad, p_pad, q_pad, _ = pk.unpack(w, out, p, q)
    compare_sample(w, out_pad, n, p_pad, q_pad, depth).assert_ok("depth 0")
    assert np.all(n == 0)


def test_packed_depth_above_k_max_is_bad():
    note("packed: a request deeper than K_max is bad data; the others verify normally")
    w = synth.random_case(5, B=6, K=5, V=900, dtype="f32", temps=(1.0,))
    depth = np.array([2, 5, 0, 4, 3, 1], np.int32)
    pk = Packed(w, depth, start=3)
    out, n, p, q = run_sample_packed(pk, w, 4)
    out_pad, p_pad, q_pad, unowned = pk.unpack(w, out, p, q)
    assert np.all(out[unowned] == -99)
    assert n[1] == -1 and np.all(out_pad[1] == -1) and np.all(p_pad[1] == 0) and np.all(q_pad[1] == 0)
    d_oracle = depth.copy()
    d_oracle[1] = -1                      # the oracle's bad request: -1 everywhere, zero p/q
    compare_sample(w, out_pad, n, p_pad, q_pad, d_oracle).assert_ok("K_max")
    pkg = Packed(w, depth)
    out, n = run_greedy_packed(pkg, 4)
    out_pad, _, _, _ = pkg.unpack(w, out)
    assert n[1] == -1 and np.all(out_pad[1] == -1)
    assert len(compare_greedy(w, out_pad, n, d_oracle)) == 0


@pytest.mark.parametrize("case", ["decreasing", "beyond_rows", "negative_start"])
def test_packed_bad_offsets(case):
    note(f"packed: offsets that are not a CSR array ({case}): every request bad, nothing else written")
    w = synth.random_case(6, B=4, K=3, V=512, dtype="bf16", temps=(1.0,))
    depth = np.array([2, 3, 1, 2], np.int32)
    pk = Packed(w, depth)
    offs = pk.offsets.copy()
    if case == "decreasing":
        offs[2] = offs[1] - 1
    elif case == "beyond_rows":
        offs[4] = pk.N + 1
    else:
        offs[0] = -1
    pk.offsets = offs
    out, n, p, q = run_sample_packed(pk, w, 3)
    assert np.all(n == -1) and np.all(out == -99) and np.all(p == -3.0) and np.all(q == -3.0)
    out, n = run_greedy_packed(pk, 3)
    assert np.all(n == -1) and np.all(out == -99)
