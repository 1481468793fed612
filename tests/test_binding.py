"""The Python binding's argument checks (no GPU needed): every tensor a call
receives, outputs and workspace included, is checked for dtype, shape and
contiguity before its pointer is taken, then for being a GPU tensor on the
call's device.  Also the host helpers that the binding forwards to the C ABI
(acceptance summary, early-exit plan)."""
import math

import pytest
import torch

sv = pytest.importorskip("draft_verification_verify_amd",
                         reason="libspecverify.so not built (run draft_verification_verify_amd/build.py)")

B, K, V = 3, 2, 16


def inputs(dtype=torch.bfloat16):
    return dict(target=torch.zeros((B, K + 1, V), dtype=dtype), draft=torch.zeros((B, K, V), dtype=dtype),
                tokens=torch.zeros((B, K), dtype=torch.int32), temperature=torch.ones(B),
                u_accept=torch.zeros((B, K)), u_sample=torch.zeros(B))


def sample(**kw):
    a = inputs()
    a.update(kw)
    return sv.verify_sample(a.pop("target"), a.pop("draft"), a.pop("tokens"), a.pop("temperature"),
                            a.pop("u_accept"), a.pop("u_sample"), **a)


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="target must be a GPU tensor"):
        sample()


@pytest.mark.parametrize("name,bad,err,msg", [
    ("out_tokens", torch.zeros((B, K), dtype=torch.int32), ValueError, "out_tokens must have shape"),
    ("out_tokens", torch.zeros((B, K + 1), dtype=torch.int64), TypeError, "out_tokens must be torch.int32"),
    ("num_accepted", torch.zeros((B + 1,), dtype=torch.int32), ValueError, "num_accepted must have shape"),
    ("p_draft", torch.zeros((B, K), dtype=torch.float64), TypeError, "p_draft must be torch.float32"),
    ("q_draft", torch.zeros((K, B)).t(), ValueError, "q_draft must be contiguous"),
    ("depth", torch.zeros((B,), dtype=torch.int64), TypeError, "depth must be torch.int32"),
])
def test_caller_outputs_are_checked_before_use(name, bad, err, msg):
    with pytest.raises(err, match=msg):
        sample(**{name: bad})


def test_wrong_shapes_and_dtypes():
    with pytest.raises(ValueError, match="3-D"):
        sample(target=torch.zeros((B, V), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="bfloat16 or float32"):
        sample(target=torch.zeros((B, K + 1, V), dtype=torch.float16))
    with pytest.raises(TypeError, match="draft must be torch.bfloat16"):
        sample(draft=torch.zeros((B, K, V), dtype=torch.float32))
    with pytest.raises(ValueError, match="u_accept must have shape"):
        sample(u_accept=torch.zeros((B, K + 1)))
    with pytest.raises(TypeError, match="torch tensor"):
        sample(tokens=[[0, 0]] * B)


def test_greedy_outputs_checked():
    with pytest.raises(ValueError, match="out_tokens must have shape"):
        sv.verify_greedy(torch.zeros((B, K + 1, V)), torch.zeros((B, K), dtype=torch.int32),
                         out_tokens=torch.zeros((B, K), dtype=torch.int32))
    with pytest.raises(ValueError, match="conf must have shape|depth_out must have shape"):
        sv.dcut_allocate(torch.zeros((B, K)), 4, depth_out=torch.zeros((B + 2,), dtype=torch.int32))
    with pytest.raises(ValueError, match="counters must have shape"):
        sv.accept_stats_update(torch.zeros(B, dtype=torch.int32), K, counters=torch.zeros(3, dtype=torch.int64))


def test_noalloc_needs_outputs():
    a = inputs()
    with pytest.raises(ValueError, match="allocates nothing"):
        sv.verify_sample_noalloc(*a.values(), out_tokens=None, num_accepted=None)


def test_workspace_checked():
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        sv._ws(dev, B, K, V, torch.zeros((64, 64), dtype=torch.uint8).t())
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        sv._ws(dev, B, K, V, torch.zeros(1 << 16, dtype=torch.uint8))


def test_accept_stats_summary_in_c():
    # counters [reached(K), accepted(K), requests, bad, sum n, sum n + 1]
    Kc = 3
    c = torch.tensor([10, 6, 0, 7, 3, 0, 10, 2, 10, 20], dtype=torch.int64)
    s = sv.accept_stats_summary(c, Kc)
    assert s["alpha"][:2] == [0.7, 0.5] and math.isnan(s["alpha"][2])
    assert s["mean_accepted"] == 1.0 and s["tau"] == 2.0 and s["bad"] == 2
    z = sv.accept_stats_summary(torch.zeros(2 * Kc + 4, dtype=torch.int64), Kc)
    assert math.isnan(z["mean_accepted"]) and math.isnan(z["tau"])
    with pytest.raises(ValueError):
        sv.accept_stats_summary(c[:-1], Kc)
