"""The allocation-free sampled verification (spec_verify_sample_noalloc,
for callers that cannot allocate device memory) against the workspace call
it shares its kernels with, through the C ABI: two calls in a row on the
library's static scratch, the second smaller than the first, each
bit-identical to spec_verify_sample on the same inputs.  Also the host-side
rejection of shapes whose workspace exceeds the static array."""
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
    import draft_verification_verify_amd  # noqa: F401


def _both(w, depth=None):
    import draft_verification_verify_amd as sv
    args = (dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature), dev(w.u_accept), dev(w.u_sample),
            dev(depth))
    ref = sv.verify_sample(*args)
    B, K = w.B, w.K
    outs = dict(out_tokens=torch.full((B, K + 1), 7, dtype=torch.int32, device="cuda"),
                num_accepted=torch.full((B,), 7, dtype=torch.int32, device="cuda"),
                p_draft=torch.full((B, K), 7.0, dtype=torch.float32, device="cuda"),
                q_draft=torch.full((B, K), 7.0, dtype=torch.float32, device="cuda"))
    got = sv.verify_sample_noalloc(*args, **outs)
    torch.cuda.synchronize()
    return [host(x) for x in ref], [host(x) for x in got]


def test_noalloc_matches_workspace_call_twice_shrinking():
    big = synth.dcut_ragged(5, T=1.0)                                        # B=64 K=16 V=128000 bf16
    small = synth.random_case(6, B=5, K=3, V=4099, dtype="f32", temps=(0.0, 0.7, 1.0), sigma=0.6)
    g = np.random.default_rng(3)
    depth = g.integers(0, small.K + 1, small.B).astype(np.int32)
    for label, w, d in (("B=64 K=16 V=128000 bf16", big, None), ("B=5 K=3 V=4099 fp32 ragged", small, depth)):
        note(f"no-alloc vs workspace call: {label}")
        ref, got = _both(w, d)
        for name, a, b in zip(("out_tokens", "num_accepted", "p_draft", "q_draft"), ref, got):
            assert np.array_equal(a, b), (label, name)
        assert np.all(got[1] >= 0)


def test_noalloc_rejects_oversized_shape():
    import draft_verification_verify_amd as sv
    note("no-alloc: a shape past the static scratch is rejected on the host")
    B, K, V = 256, 64, 128000
    assert sv.workspace_size(B, K, V) > sv.NOALLOC_SCRATCH_BYTES
    t = torch.empty((B, K + 1, 8), dtype=torch.bfloat16, device="cuda")   # never read
    st = sv.lib.spec_verify_sample_noalloc(t.data_ptr(), t.data_ptr(), 1, t.data_ptr(), None, t.data_ptr(),
                                           t.data_ptr(), t.data_ptr(), B, K, V, t.data_ptr(), t.data_ptr(),
                                           None, None, None)
    assert st == 2
    assert "static array" in sv.lib.spec_verify_last_error().decode()
