"""GPU parity of draft statistics taken at each request's own temperature
(spec_draft_confidence_stats_t) and of their reuse by spec_verify_sample_reuse,
through the C ABI.

The statistics of draft row (b, k) at temperature T are the row's max M and
sum over v of exp((v - M) / T), the softmax normaliser the oracle's softmax
returns; each record carries the bits of the T it was taken at.  The
confidence D-cut ranks by stays the T = 1 value.  A sampled request reuses
the statistics when its record's temperature matches its own (then its draft
rows are not streamed), and is verified as by spec_verify_sample otherwise;
either way every output must follow the oracle's verify_sample rules."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import Tally, compare_sample, dev, host

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


def stats_t(w, max_depth=None, temperature=None):
    import draft_verification_verify_amd as sv
    T = w.temperature if temperature is None else temperature
    conf, st = sv.draft_confidence_stats(dev(w.draft), dev(max_depth), temperature=dev(T))
    torch.cuda.synchronize()
    return conf, st


def reuse(w, st, depth=None):
    import draft_verification_verify_amd as sv
    out, n, p, q = sv.verify_sample_reuse(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                          dev(w.u_accept), dev(w.u_sample), st, dev(depth))
    torch.cuda.synchronize()
    return host(out), host(n), host(p), host(q)


def check_stats(w, conf, st, max_depth=None):
    """Records against the oracle's softmax normaliser at each request's
    statistics temperature, and the T = 1 confidence against the oracle's."""
    import draft_verification_verify_amd as sv
    mx, sm, tt = (host(t) for t in sv.row_stat_fields(st))
    conf_o = oracle.draft_confidence(w.draft, max_depth)
    c = host(conf)
    m = conf_o > 0
    assert np.all(c[~m] == 0) and np.max(np.abs(c[m] - conf_o[m]) / conf_o[m]) < 2e-6
    K = w.K
    md = np.full(w.B, K) if max_depth is None else np.asarray(max_depth)
    for b in range(w.B):
        T = float(w.temperature[b])
        Ts = T if (T > 0 and np.isfinite(T) and T != 1.0) else 1.0
        for k in range(K):
            if k >= md[b]:
                assert np.isnan(mx[b, k]) and np.isnan(sm[b, k])
                continue
            assert tt[b, k] == np.float32(Ts), (b, k, tt[b, k], Ts)
            _, M, S = oracle.softmax(w.draft[b, k], Ts)
            assert mx[b, k] == np.float32(M), (b, k)
            assert abs(sm[b, k] - S) <= 2e-6 * S, (b, k, sm[b, k], S, Ts)


def test_statistics_at_each_temperature():
    note("statistics at T in {0, 0.05, 0.5, 0.7, 1, 1.6, 10} (bf16 V=4099, K=5, ragged max_depth)")
    temps = np.array([0.0, 0.05, 0.5, 0.7, 1.0, 1.6, 10.0, 0.7], np.float32)
    w = synth.random_case(31, B=temps.size, K=5, V=4099, dtype="bf16", temperature=temps, sigma=0.6)
    max_depth = np.array([5, 5, 3, 0, 5, 1, 5, 4], np.int32)
    conf, st = stats_t(w, max_depth)
    check_stats(w, conf, st, max_depth)


def test_statistics_temperature_extremes_fp32():
    note("statistics at T from 1e-40 to 3e38 (fp32 V=7000): the second sum's scale shifts below T = 1e-30")
    temps = np.array([1e-40, 1e-32, 1e-6, 3e-3, 1e3, 1e30, 3e38, 1.0], np.float32)
    w = synth.random_case(32, B=temps.size, K=3, V=7000, dtype="f32", temperature=temps, sigma=0.5)
    conf, st = stats_t(w)
    check_stats(w, conf, st)


def test_reuse_any_temperature_mixed_fp32_full_size():
    note("mixed fp32 B=64 V=152064, T in {0, 0.7, 1}: statistics at each T -> dcut_allocate(512) -> reuse")
    import draft_verification_verify_amd as sv
    w = synth.mixed(0)
    conf, st = stats_t(w, w.max_depth)
    # the T = 1 confidence is the same bits as the single-statistic pass's
    conf1 = sv.draft_confidence(dev(w.draft), dev(w.max_depth))
    assert np.array_equal(host(conf), host(conf1))
    depth = oracle.dcut_allocate(oracle.draft_confidence(w.draft, w.max_depth), w.budget, w.max_depth)
    out, n, p, q = reuse(w, st, depth)
    compare_sample(w, out, n, p, q, depth).assert_ok("reuse at every T")
    assert np.all(n >= 0)


@pytest.mark.parametrize("dtype,V", [("f32", 7), ("bf16", 64), ("f32", 1000), ("bf16", 4099), ("f32", 9001)])
@pytest.mark.parametrize("K", [1, 3, 16])
def test_reuse_any_temperature_fuzz(dtype, V, K):
    note(f"reuse at each request's T, fuzz {dtype} V={V} K={K}")
    B = 8
    w = synth.random_case(V * 13 + K, B=B, K=K, V=V, dtype=dtype, temps=(0.0, 0.4, 0.7, 1.0, 1.6), sigma=0.6)
    g = np.random.default_rng(V * 7 + K)
    depth = g.integers(0, K + 1, B).astype(np.int32)
    _, st = stats_t(w)
    tal = Tally()
    out, n, p, q = reuse(w, st, depth)
    compare_sample(w, out, n, p, q, depth, tal)
    out, n, p, q = reuse(w, st)
    compare_sample(w, out, n, p, q, None, tal)
    tal.assert_ok(f"reuse any T {dtype} V={V} K={K}")


def test_statistics_at_another_temperature_are_not_reused():
    note("records taken at T = 1 given to requests at 0.7 and 1.6: their draft rows are streamed instead")
    import draft_verification_verify_amd as sv
    w = synth.random_case(33, B=6, K=4, V=3000, dtype="f32", temps=(0.7, 1.0, 1.6), sigma=0.6)
    _, st1 = sv.draft_confidence_stats(dev(w.draft))      # all at T = 1
    out, n, p, q = reuse(w, st1)
    compare_sample(w, out, n, p, q).assert_ok("T = 1 records, mixed requests")
    _, stt = stats_t(w, temperature=np.full(6, 0.7, np.float32))   # all at 0.7
    out, n, p, q = reuse(w, stt)
    compare_sample(w, out, n, p, q).assert_ok("T = 0.7 records, mixed requests")


def test_record_at_another_temperature_after_the_first_is_bad():
    note("a request whose first record matches its T but a later one does not is bad data")
    w = synth.random_case(34, B=3, K=4, V=800, dtype="f32", temps=(0.7,), sigma=0.6)
    _, st = stats_t(w)
    st2 = st.clone()
    f = st2.view(torch.float32)
    f[1, 2, 1] = 1.0                                   # request 1, row 2: taken at T = 1
    out, n, p, q = reuse(w, st2)
    assert n[1] == -1 and np.all(out[1] == -1)
    ok = np.array([0, 2])
    sub = synth.Workload(w.name, w.dtype, w.target[ok], w.draft[ok], w.tokens[ok], w.temperature[ok],
                         w.u_accept[ok], w.u_sample[ok], w.max_depth[ok])
    compare_sample(sub, out[ok], n[ok], p[ok], q[ok]).assert_ok("the other requests")
