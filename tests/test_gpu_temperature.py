"""GPU parity across the whole temperature range and for rows with large
logits, through the C ABI.

The contract accepts every finite T > 0.  The row statistics form each
exponent as (v - M) / T on a scale of about log2(e)/T, so small T and large
|M| stress the same arithmetic: the rounding offset of M * log2(e)/T grows
with both.  These cases check the one-pass, early-exit and draft-statistics
reuse calls (statistics at T = 1 and at each request's temperature) at T
from 1e-45 (an fp32 denormal) to 3.4e38 on bf16 V=128000 and fp32 V=152064
rows, and rows shifted by a constant of 1e5 to 1e6 (the
softmax is shift invariant; the stored logits are rounded after the shift,
and the oracle sees the same bytes)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import Tally, compare_sample, dev, host, run_sample, run_sample_reuse

pytestmark = pytest.mark.gpu

SWEEP = [1e-45, 1e-40, 1e-30, 1e-6, 1e-5, 3e-5, 1e-4, 1e-3, 0.01, 0.1, 10.0, 1e3, 1e6, 1e30, 3.4e38]


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    import draft_verification_verify_amd  # noqa: F401


def sweep_case(dtype, V, seed, K=3, shift=0.0, temps=SWEEP, sigma=0.5):
    T = np.repeat(np.asarray(temps, np.float32), 2)
    return synth.random_case(seed, B=T.size, K=K, V=V, dtype=dtype, sigma=sigma, shift=shift, temperature=T)


def run_early_exit(w, ends):
    import draft_verification_verify_amd as sv
    out, n, p, q = sv.verify_sample_early_exit(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                               dev(w.u_accept), dev(w.u_sample), ends=ends)
    torch.cuda.synchronize()
    return host(out), host(n), host(p), host(q)


def compare_early_exit(w, out, n, p, q):
    """Tokens and counts follow the one-pass rules; p/q are compared at the
    positions the early-exit reading reads (k <= min(n, d - 1))."""
    ora = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept, w.u_sample)
    tal = compare_sample(w, out, n, None, None, ora=ora)
    ee = oracle.verify_early_exit(w.target, w.tokens, w.draft, w.temperature, w.u_accept, w.u_sample)
    tal.max_pq_err = max(float(np.max(np.abs(p - ee["p_draft"]))), float(np.max(np.abs(q - ee["q_draft"]))))
    return tal


@pytest.mark.parametrize("dtype,V", [("bf16", 128000), ("f32", 152064)])
def test_sample_temperature_sweep(dtype, V):
    note(f"sample temperature sweep {dtype} V={V}: T from 1e-45 to 3.4e38")
    tal = Tally()
    for seed in range(2):
        w = sweep_case(dtype, V, 100 + seed)
        out, n, p, q = run_sample(w)
        compare_sample(w, out, n, p, q, tally=tal)
        assert np.all(n >= 0), n
    tal.assert_ok(f"sweep {dtype}")


@pytest.mark.parametrize("dtype,V", [("bf16", 128000), ("f32", 152064)])
def test_early_exit_temperature_sweep(dtype, V):
    note(f"early-exit temperature sweep {dtype} V={V}, window ends [1, 3]")
    w = sweep_case(dtype, V, 200)
    out, n, p, q = run_early_exit(w, [1, 3])
    compare_early_exit(w, out, n, p, q).assert_ok(f"early exit sweep {dtype}")


@pytest.mark.parametrize("dtype,V", [("bf16", 128000), ("f32", 152064)])
def test_reuse_temperature_sweep(dtype, V):
    note(f"draft-statistics reuse with T from 1e-45 to 3.4e38 (only T = 1 requests reuse) {dtype} V={V}")
    w = sweep_case(dtype, V, 300, temps=SWEEP + [1.0])
    out, n, p, q = run_sample_reuse(w)
    compare_sample(w, out, n, p, q).assert_ok(f"reuse sweep {dtype}")


@pytest.mark.parametrize("shift", [1e5, 1e6, -1e6])
def test_sample_shifted_rows_fp32(shift):
    note(f"fp32 V=152064 rows shifted by {shift:g}: one pass, early exit and reuse at T in (1, 1e-3, 1e-4)")
    w = sweep_case("f32", 152064, 400, K=4, shift=shift, temps=[1.0, 1e-3, 1e-4, 1.0])
    tal = Tally()
    out, n, p, q = run_sample(w)
    compare_sample(w, out, n, p, q, tally=tal)
    out, n, p, q = run_sample_reuse(w)
    compare_sample(w, out, n, p, q, tally=tal)
    tal.assert_ok(f"shift {shift:g}")
    out, n, p, q = run_early_exit(w, [2, 4])
    compare_early_exit(w, out, n, p, q).assert_ok(f"shift {shift:g} early exit")
    assert np.all(n >= 0)


@pytest.mark.parametrize("shift", [1e5, -1e6])
def test_confidence_shifted_rows_fp32(shift):
    note(f"draft confidence of fp32 V=152064 rows shifted by {shift:g}")
    import draft_verification_verify_amd as sv
    w = sweep_case("f32", 152064, 500, K=4, shift=shift, temps=[1.0] * 4)
    conf_g = host(sv.draft_confidence(dev(w.draft)))
    conf_o = oracle.draft_confidence(w.draft)
    assert np.max(np.abs(conf_g - conf_o) / conf_o) < 2e-6


@pytest.mark.parametrize("dtype,V", [("bf16", 128000), ("f32", 152064)])
def test_reuse_any_temperature_sweep(dtype, V):
    note(f"draft-statistics reuse taken at each request's temperature, T from 1e-45 to 3.4e38, {dtype} V={V}")
    import draft_verification_verify_amd as sv
    w = sweep_case(dtype, V, 310, temps=SWEEP + [1.0])
    T = dev(w.temperature)
    _, st = sv.draft_confidence_stats(dev(w.draft), None, temperature=T, want_conf=False)
    out, n, p, q = sv.verify_sample_reuse(dev(w.target), dev(w.draft), dev(w.tokens), T, dev(w.u_accept),
                                          dev(w.u_sample), st)
    torch.cuda.synchronize()
    out, n, p, q = host(out), host(n), host(p), host(q)
    compare_sample(w, out, n, p, q).assert_ok(f"reuse at each temperature {dtype}")
    assert np.all(n >= 0), n
