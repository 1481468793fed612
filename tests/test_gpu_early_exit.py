"""GPU parity of spec_verify_greedy_early_exit / spec_verify_sample_early_exit
against the oracle's early-exit verification, through the C ABI.

Greedy requests are compared bit-exactly.  Sampled requests use the bands
of the one-pass parity tests (decision band 1e-5 around min(1, p/q), CDF
band 1e-6 for the emitted token); p_draft / q_draft within 1e-6 where both
sides stopped at the same position.  Rows, tokens and uniforms after the
oracle's stopping position are poisoned in some cases to show that they are
not read."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import Tally, compare_sample, dev, host, run_greedy, run_sample

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


def _win(window):
    """int: fixed windows of that many positions; list: window ends; None: the default."""
    if isinstance(window, (list, tuple)):
        return {"ends": list(window)}
    return {"window": window}


def run_ee_greedy(w, depth=None, window=4, tokens=None, target=None):
    import draft_verification_verify_amd as sv
    tok = w.tokens if tokens is None else tokens
    tgt = w.target if target is None else target
    out, n = sv.verify_greedy_early_exit(dev(tgt), dev(tok), dev(depth), **_win(window))
    torch.cuda.synchronize()
    return host(out), host(n)


def run_ee_sample(w, depth=None, window=4):
    import draft_verification_verify_amd as sv
    out, n, p, q = sv.verify_sample_early_exit(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                               dev(w.u_accept), dev(w.u_sample), dev(depth), **_win(window))
    torch.cuda.synchronize()
    return host(out), host(n), host(p), host(q)


def oracle_ee_sample(w, depth=None):
    return oracle.verify_early_exit(w.target, w.tokens, w.draft, w.temperature, w.u_accept, w.u_sample, depth)


def compare_ee_sample(w, res, ora, depth=None, tally=None):
    """Decisions and tokens with the one-pass bands; the decision band reads
    the ratio from the oracle's own p/q at the positions it read."""
    out, n, p, q = res
    tally = tally or Tally()
    po, qo = ora["p_draft"].astype(np.float64), ora["q_draft"].astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(qo > 0, np.minimum(1.0, po / qo), np.where(po > 0, 1.0, 0.0))
    compare_sample(w, out, n, None, None, depth, tally, dict(ora, ratio=ratio))
    same = n == ora["n"]
    if np.any(same):
        tally.max_pq_err = max(tally.max_pq_err,
                               float(np.max(np.abs(p[same] - ora["p_draft"][same]), initial=0.0)),
                               float(np.max(np.abs(q[same] - ora["q_draft"][same]), initial=0.0)))
    for b in np.nonzero(~same)[0]:
        m = int(min(n[b], ora["n"][b]))
        if m >= 0:
            tally.max_pq_err = max(tally.max_pq_err, float(np.max(np.abs(p[b, :m] - ora["p_draft"][b, :m]),
                                                                  initial=0.0)))
    return tally


def poison_after(w, depth, n_stop):
    """Copy of w with NaN rows, out-of-range tokens and invalid uniforms at
    every position after each request's stopping position."""
    t, d, tok, ua = w.target.copy(), w.draft.copy(), w.tokens.copy(), w.u_accept.copy()
    nan = synth.to_bf16_bits(np.array([np.nan], np.float32))[0] if t.dtype == np.uint16 else np.nan
    dd = np.full(w.B, w.K) if depth is None else depth
    for b in range(w.B):
        nb = int(n_stop[b])
        if 0 <= nb < int(dd[b]):
            t[b, nb + 1:, :] = nan
            d[b, nb + 1:, :] = nan
            tok[b, nb + 1:] = -3
            ua[b, nb + 1:] = 2.0
    return synth.Workload(w.name + "_poisoned", w.dtype, t, d, tok, w.temperature, ua, w.u_sample, w.max_depth)


# ---------------------------------------------------------------- greedy ----

@pytest.mark.parametrize("dtype,V", [("bf16", 1), ("f32", 7), ("bf16", 63), ("f32", 1000), ("bf16", 4099),
                                     ("bf16", 70001)])
@pytest.mark.parametrize("K", [0, 1, 5, 16])
def test_ee_greedy_fuzz_shapes(dtype, V, K):
    note(f"early-exit greedy fuzz {dtype} V={V} K={K}")
    B = 7
    w = synth.random_case(V * 13 + K, B=B, K=K, V=V, dtype=dtype, temps=(0.0,), sigma=0.15)
    depth = np.random.default_rng(V + 5 * K).integers(0, K + 1, B).astype(np.int32)
    ora = oracle.verify_early_exit(w.target, w.tokens, depth=depth)
    one_out, one_n = run_greedy(w, depth)
    for window in (1, 2, 3, 16, 1000, None, [1, max(K, 1)], [2, 3, K + 4]):
        out, n = run_ee_greedy(w, depth, window)
        assert np.array_equal(n, ora["n"]) and np.array_equal(out, ora["out"]), (window, n, ora["n"])
        assert np.array_equal(n, one_n) and np.array_equal(out, one_out)


def test_ee_greedy_nothing_read_after_stop():
    note("early-exit greedy: poisoned rows after the stop")
    w = synth.random_case(3, B=16, K=12, V=5003, dtype="bf16", temps=(0.0,), sigma=0.15)
    depth = np.random.default_rng(1).integers(0, w.K + 1, w.B).astype(np.int32)
    ora = oracle.verify_early_exit(w.target, w.tokens, depth=depth)
    assert np.any(ora["n"] < depth)
    wp = poison_after(w, depth, ora["n"])
    orap = oracle.verify_early_exit(wp.target, wp.tokens, depth=depth)
    assert np.array_equal(orap["out"], ora["out"]) and np.array_equal(orap["n"], ora["n"])
    for window in (1, 4, 12):
        out, n = run_ee_greedy(wp, depth, window)
        assert np.array_equal(n, ora["n"]) and np.array_equal(out, ora["out"]), window
    # the one-pass call reads the whole window and reports those requests as bad
    _, n1 = run_greedy(wp, depth)
    assert np.all(n1[ora["n"] < depth] == -1)


def test_ee_greedy_bad_data_before_stop():
    note("early-exit greedy: bad data at or before the stop, and a bad bonus row")
    g = np.random.default_rng(9)
    B, K, V = 5, 6, 3000
    target = g.standard_normal((B, K + 1, V)).astype(np.float32)
    am = np.argmax(target, axis=2).astype(np.int32)
    tokens = am[:, :K].copy()
    tokens[:, 3] = (am[:, 3] + 1) % V           # every request rejects at position 3
    target[0, 1, 17] = np.nan                   # before the stop
    target[1, 3, :] = -np.inf                   # at the stop
    tokens[2, 4] = V + 1                        # after the stop: never read
    target[2, 5, :] = np.nan                    # after the stop: never read
    tokens[3, 3] = am[3, 3]                     # request 3 accepts everything ...
    target[3, K, 2] = np.inf                    # ... and its bonus row is bad
    tokens[4, 0] = -1                           # position 0 token out of range
    w = synth.Workload("ee_bad", "f32", target, target[:, :K].copy(), tokens, np.zeros(B, np.float32),
                       np.zeros((B, K), np.float32), np.zeros(B, np.float32), np.full(B, K, np.int32))
    ora = oracle.verify_early_exit(target, tokens)
    assert ora["n"].tolist() == [-1, -1, 3, -1, -1]
    for window in (1, 2, 4, 6):
        out, n = run_ee_greedy(w, None, window)
        assert np.array_equal(n, ora["n"]) and np.array_equal(out, ora["out"]), window


def test_ee_greedy_full_size():
    note("early-exit greedy dcut_ragged B=64 K=16 V=128000 bf16, dense and ragged")
    w = synth.dcut_ragged(0, T=0.0)
    ora = oracle.verify_early_exit(w.target, w.tokens)
    for window in (2, 4, 8):
        out, n = run_ee_greedy(w, None, window)
        assert np.array_equal(n, ora["n"]) and np.array_equal(out, ora["out"]), window
    depth = np.random.default_rng(2).integers(1, w.K + 1, w.B).astype(np.int32)
    ora = oracle.verify_early_exit(w.target, w.tokens, depth=depth)
    out, n = run_ee_greedy(w, depth, 4)
    assert np.array_equal(n, ora["n"]) and np.array_equal(out, ora["out"])


# --------------------------------------------------------------- sampled ----

@pytest.mark.parametrize("dtype,V", [("bf16", 1), ("f32", 7), ("bf16", 64), ("f32", 1000), ("bf16", 4099),
                                     ("f32", 9001), ("bf16", 70001)])
@pytest.mark.parametrize("K", [0, 1, 4, 16])
def test_ee_sample_fuzz_shapes(dtype, V, K):
    note(f"early-exit sample fuzz {dtype} V={V} K={K}")
    B = 8
    w = synth.random_case(V * 5 + K, B=B, K=K, V=V, dtype=dtype, temps=(0.0, 0.7, 1.0, 1.6), sigma=0.5)
    depth = np.random.default_rng(V * 2 + K).integers(0, K + 1, B).astype(np.int32)
    tal = Tally()
    for dep in (depth, None):
        ora = oracle_ee_sample(w, dep)
        for window in (1, 3, 16, None, [1, max(K, 1)], [2, 3, K + 4]):
            compare_ee_sample(w, run_ee_sample(w, dep, window), ora, dep, tal)
    tal.assert_ok(f"{dtype} V={V} K={K}")


def test_ee_sample_nothing_read_after_stop():
    note("early-exit sample: poisoned rows, tokens and uniforms after the stop")
    w = synth.random_case(4, B=24, K=10, V=9001, dtype="f32", temps=(0.0, 0.8, 1.0), sigma=0.9)
    depth = np.random.default_rng(3).integers(0, w.K + 1, w.B).astype(np.int32)
    ora = oracle_ee_sample(w, depth)
    assert np.any((ora["n"] >= 0) & (ora["n"] < depth))
    wp = poison_after(w, depth, ora["n"])
    orap = oracle_ee_sample(wp, depth)
    for key in ("out", "n", "p_draft", "q_draft"):
        assert np.array_equal(orap[key], ora[key])
    tal = Tally()
    for window in (1, 2, 5, 10):
        compare_ee_sample(wp, run_ee_sample(wp, depth, window), ora, depth, tal)
    tal.assert_ok("poisoned")
    # the one-pass call reads the whole window, so most of those requests are
    # bad there (not all: a sampled request stopping at d-1 reads no row
    # after its stop in either call)
    _, n1, _, _ = run_sample(wp, depth)
    full = oracle.verify_sample(wp.target, wp.draft, wp.tokens, wp.temperature, wp.u_accept, wp.u_sample, depth)
    bad1 = full["n"] == -1
    assert np.sum(bad1 & (ora["n"] >= 0)) >= 5 and np.all(n1[bad1] == -1)


def test_ee_sample_bad_inputs():
    note("early-exit sample: bad data before, at and after the stop")
    w = synth.random_case(1, B=8, K=4, V=640, dtype="f32", temps=(1.0,), sigma=3.0)
    t, d = w.target.copy(), w.draft.copy()
    tok, ua, us, T = w.tokens.copy(), w.u_accept.copy(), w.u_sample.copy(), w.temperature.copy()
    ua[:, 0] = 0.0               # position 0 accepts unless its data is bad
    ua[:, 1] = 0.999999          # position 1 rejects unless p/q >= 1 there
    tok[0, 0] = -1               # position 0: bad
    ua[1, 0] = 1.0               # position 0: bad uniform
    T[2] = -0.5                  # bad temperature
    d[3, 3, :] = np.nan          # after a stop at 1: never read (unless accepted)
    d[4, 0, 3] = np.nan          # position 0: bad draft row
    us[5] = 1.5                  # bad draw uniform: read by every sampled request
    t[6, 1, :] = -np.inf         # position 1: bad target row
    w2 = synth.Workload("ee_bad", "f32", t, d, tok, T, ua, us, w.max_depth)
    ora = oracle_ee_sample(w2)
    assert ora["n"].tolist()[:3] == [-1, -1, -1] and ora["n"][4] == -1 and ora["n"][5] == -1
    assert ora["n"][6] == -1
    tal = Tally()
    for window in (1, 2, 4):
        res = run_ee_sample(w2, None, window)
        compare_ee_sample(w2, res, ora, None, tal)
        assert np.all(res[2][ora["n"] == -1] == 0) and np.all(res[0][ora["n"] == -1] == -1)
    tal.assert_ok("bad inputs")


@pytest.mark.parametrize("window", [1, 2, 4, 8, 16, None, [1, 16], [2, 6, 16]])
def test_ee_sample_full_size(window):
    note(f"early-exit sample dcut_ragged B=64 K=16 V=128000 bf16 T=1, window {window}")
    w = synth.dcut_ragged(0, T=1.0)
    ora = oracle_ee_sample(w)
    res = run_ee_sample(w, None, window)
    tal = compare_ee_sample(w, res, ora)
    tal.assert_ok(f"window {window}")
    # the one-pass call on the same data commits the same tokens
    out1, n1, _, _ = run_sample(w)
    diff = np.nonzero((n1 != res[1]) | np.any(out1 != res[0], axis=1))[0]
    assert len(diff) <= tal.excused


def test_ee_mixed_fp32_full_size():
    note("early-exit sample mixed fp32 B=64 V=152064, depth = K_b (padding rows NaN), windows 3 and 16")
    w = synth.mixed(0)
    depth = w.max_depth.copy()
    ora = oracle_ee_sample(w, depth)
    assert np.all(ora["n"] >= 0)
    tal = Tally()
    for window in (3, 16):
        compare_ee_sample(w, run_ee_sample(w, depth, window), ora, depth, tal)
    tal.assert_ok("mixed")


def test_ee_maximum_sizes():
    note("early-exit at the limits: B=4096 (K=3, V=17) and K=1024 (B=2, V=33)")
    w = synth.random_case(31, B=4096, K=3, V=17, dtype="f32", temps=(0.0, 1.0), sigma=0.6)
    ora = oracle_ee_sample(w)
    tal = Tally()
    for window in (1, 3):
        compare_ee_sample(w, run_ee_sample(w, None, window), ora, None, tal)
    og = oracle.verify_early_exit(w.target, w.tokens)
    out, n = run_ee_greedy(w, None, 2)
    assert np.array_equal(n, og["n"]) and np.array_equal(out, og["out"])
    # low draft noise: long accepted prefixes over many windows
    w2 = synth.random_case(32, B=2, K=1024, V=33, dtype="bf16", temps=(1.0,), sigma=0.05)
    ora2 = oracle_ee_sample(w2)
    assert ora2["n"].max() > 20
    for window in (7, 100, 1024):
        compare_ee_sample(w2, run_ee_sample(w2, None, window), ora2, None, tal)
    tal.assert_ok("limits")


def test_ee_workspace_reuse_and_alternating_calls():
    note("early-exit: one workspace across one-pass and early-exit calls of different shapes")
    import draft_verification_verify_amd as sv
    ws = torch.empty(sv.workspace_size(64, 16, 128000), dtype=torch.uint8, device="cuda")
    w1 = synth.random_case(11, B=64, K=16, V=4099, dtype="bf16", temps=(0.0, 1.0), sigma=0.4)
    w2 = synth.random_case(12, B=9, K=5, V=70001, dtype="f32", temps=(0.7, 1.0), sigma=0.4)
    o1, o2 = oracle_ee_sample(w1), oracle_ee_sample(w2)
    tal = Tally()
    for rep in range(2):
        for w, o in ((w1, o1), (w2, o2)):
            res = sv.verify_sample_early_exit(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                              dev(w.u_accept), dev(w.u_sample), window=3, workspace=ws)
            torch.cuda.synchronize()
            compare_ee_sample(w, tuple(host(x) for x in res), o, None, tal)
            sv.verify_sample(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                             dev(w.u_accept), dev(w.u_sample), workspace=ws)
    torch.cuda.synchronize()
    tal.assert_ok("alternating")
