"""HIP-graph capture of the verification calls (through torch.cuda.CUDAGraph,
which captures the launches the library enqueues on the current stream).

The kernels are deterministic (static schedules, no atomics on the verify
path), so every replay must reproduce the eager call bit for bit.  Replays
are separated by eager work on the same buffers (outputs overwritten, an
input changed in place) and by synchronisations, and every replay is
checked."""
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


def test_graph_replays_match_eager():
    import draft_verification_verify_amd as sv
    note("graph capture: confidence -> dcut_allocate -> sample verify, and an early-exit verify")
    w = synth.random_case(21, B=16, K=8, V=40000, dtype="bf16", temps=(0.0, 0.7, 1.0), sigma=0.5)
    B, K, V = w.B, w.K, w.V
    t, d, tok = dev(w.target), dev(w.draft), dev(w.tokens)
    T, ua, us = dev(w.temperature), dev(w.u_accept), dev(w.u_sample)
    ws1 = torch.empty(sv.workspace_size(B, K, V), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws1)
    conf = torch.empty((B, K), dtype=torch.float32, device="cuda")
    depth = torch.empty((B,), dtype=torch.int32, device="cuda")
    outs = [torch.empty((B, K + 1), dtype=torch.int32, device="cuda") for _ in range(2)]
    ns = [torch.empty((B,), dtype=torch.int32, device="cuda") for _ in range(2)]
    ps = [torch.empty((B, K), dtype=torch.float32, device="cuda") for _ in range(4)]

    def body():
        sv.draft_confidence(d, conf=conf, workspace=ws1)
        sv.dcut_allocate(conf, 3 * B, depth_out=depth)
        sv.verify_sample(t, d, tok, T, ua, us, depth, out_tokens=outs[0], num_accepted=ns[0],
                         p_draft=ps[0], q_draft=ps[1], workspace=ws1)
        sv.verify_sample_early_exit(t, d, tok, T, ua, us, window=3, out_tokens=outs[1], num_accepted=ns[1],
                                    p_draft=ps[2], q_draft=ps[3], workspace=ws2)

    def snapshot():
        torch.cuda.synchronize()
        return [host(x).copy() for x in [conf, depth] + outs + ns + ps]

    # eager reference (also warms the library's per-device caches)
    body()
    ref = snapshot()
    us_alt = torch.rand(B, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3)) * 0.999
    us_orig = us.clone()
    us.copy_(us_alt)
    body()
    ref_alt = snapshot()
    us.copy_(us_orig)
    assert np.all(ref[4] >= 0) and np.all(ref[5] >= 0)   # num_accepted: every request valid
    assert not np.array_equal(ref[2], ref_alt[2])         # the changed draw uniforms change tokens

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    for rep in range(4):
        for x in outs + ns + ps:
            x.fill_(-7)
        conf.zero_()
        alt = rep % 2 == 1
        us.copy_(us_alt if alt else us_orig)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        want = ref_alt if alt else ref
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"replay {rep}: buffer {i} differs from the eager call"
    us.copy_(us_orig)
    # eager work after the replays still gives the eager result
    body()
    got = snapshot()
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
