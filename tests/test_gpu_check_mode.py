"""Check mode (SPECVERIFY_CHECK=1): verify calls and dcut_allocate wait for
their work and return SV_ERR_BAD_INPUT when a request reported bad data;
without it the same calls succeed and report the request in num_accepted."""
import sys

import numpy as np
import pytest
import torch

import synth
from parity import dev, host

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_verify_amd  # noqa: F401  (fails loudly if the library is missing)


def test_check_mode_reports_bad_requests(monkeypatch):
    import draft_verification_verify_amd as sv
    note("check mode: bad token at position 0 of request 3")
    w = synth.random_case(2, B=6, K=4, V=3000, dtype="f32", temps=(0.0, 1.0), sigma=0.5)
    tok_bad = w.tokens.copy()
    tok_bad[3, 0] = -1          # read by every call: position 0
    t, d, T, ua, us = dev(w.target), dev(w.draft), dev(w.temperature), dev(w.u_accept), dev(w.u_sample)
    good, bad = dev(w.tokens), dev(tok_bad)
    calls = {
        "spec_verify_greedy": lambda tk: sv.verify_greedy(t, tk),
        "spec_verify_sample": lambda tk: sv.verify_sample(t, d, tk, T, ua, us),
        "spec_verify_greedy_early_exit": lambda tk: sv.verify_greedy_early_exit(t, tk, window=2),
        "spec_verify_sample_early_exit": lambda tk: sv.verify_sample_early_exit(t, d, tk, T, ua, us, window=2),
    }
    monkeypatch.setenv("SPECVERIFY_CHECK", "1")
    for name, fn in calls.items():
        res = fn(good)
        assert np.all(host(res[1]) >= 0), name
        with pytest.raises(sv.SpecVerifyError) as e:
            fn(bad)
        assert e.value.status == 5 and name in str(e.value) and "request 3" in str(e.value), str(e.value)
    conf = torch.full((6, 4), 0.5, device="cuda")
    assert np.all(host(sv.dcut_allocate(conf, 12)) >= 1)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.dcut_allocate(conf, 12, dev(np.array([4, 4, 9, 4, 4, 4], np.int32)))   # max_depth 9 > K
    assert e.value.status == 5 and "request 2" in str(e.value)
    monkeypatch.delenv("SPECVERIFY_CHECK")
    for name, fn in calls.items():
        n = host(fn(bad)[1])
        torch.cuda.synchronize()
        assert n[3] == -1 and np.all(np.delete(n, 3) >= 0), name


def test_read_ceiling_sizes():
    import draft_verification_verify_amd as sv
    note("read ceiling: whole blocks, a partial block and a vector tail")
    for nbytes in (16, 4096, 4096 + 48, 8 * 4096 * 1024 + 16 * 37):
        buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        sink = torch.full((1,), 5, dtype=torch.int32, device="cuda")
        sv.read_ceiling(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 5     # a fold of zeros never matches the stored value
