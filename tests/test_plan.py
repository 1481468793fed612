"""spec_early_exit_plan (host computation, no GPU): the window ends it returns
minimise the expected cost over every list of ends, checked by brute force
over all lists for small K, plus closed-form cases and argument checks."""
import ctypes
import itertools

import numpy as np
import pytest

sv = pytest.importorskip("draft_verification_verify_amd",
                         reason="libspecverify.so not built (run draft_verification_verify_amd/build.py)")


def plan_cost(alpha, c, ends):
    live = np.concatenate([[1.0], np.cumprod(alpha)])
    cost, lo = 0.0, 0
    for e in ends:
        cost += c + live[lo] * (e - lo)
        lo = e
    return cost


def all_plans(K):
    for r in range(K):
        for cut in itertools.combinations(range(1, K), r):
            yield list(cut) + [K]


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8])
def test_plan_is_optimal_by_brute_force(K):
    g = np.random.default_rng(K)
    for trial in range(40):
        alpha = g.random(K) ** g.uniform(0.2, 3.0)
        c = float(g.choice([0.0, 0.3, 1.0, 2.5, 7.0]))
        got = sv.early_exit_plan(alpha, c)
        assert got[-1] == K and all(b > a for a, b in zip(got, got[1:])) and got[0] >= 1
        costs = sorted((plan_cost(alpha, c, p), p) for p in all_plans(K))
        assert plan_cost(alpha, c, got) <= costs[0][0] * (1 + 1e-12) + 1e-12
        if len(costs) > 1 and costs[1][0] - costs[0][0] > 1e-9:
            assert got == costs[0][1]


def test_plan_closed_forms():
    K = 16
    assert sv.early_exit_plan([1.0] * K, 2.5) == [K]            # nothing stops: one window
    assert sv.early_exit_plan([0.0] * K, 2.5) == [1, K]         # everything stops at position 0
    assert sv.early_exit_plan([0.0] * K, 20.0) == [K]           # windows dearer than the whole block
    assert sv.early_exit_plan([0.5] * K, 0.0) == list(range(1, K + 1))   # free windows: one per position
    assert sv.early_exit_plan([], 3.0) == [1]                   # K = 0
    assert sv.early_exit_plan([float("nan")] * 3, 1.0) == [1, 3]   # unreached positions count as 0
    assert sv.early_exit_plan([0.9, float("nan"), 0.7], 1.0) == sv.early_exit_plan([0.9, 0.0, 0.7], 1.0)


def test_plan_argument_errors():
    L = sv.lib
    a = (ctypes.c_double * 3)(0.5, 0.5, 0.5)
    ends = (ctypes.c_int32 * 3)()
    n = ctypes.c_int32(0)
    A, E, N = (ctypes.cast(x, ctypes.c_void_p) for x in (a, ends, ctypes.pointer(n)))
    assert L.spec_early_exit_plan(A, 3, 1.0, E, N) == 0 and n.value >= 1
    assert L.spec_early_exit_plan(A, 3, 1.0, None, N) == 1
    assert L.spec_early_exit_plan(A, 3, 1.0, E, None) == 1
    assert L.spec_early_exit_plan(None, 3, 1.0, E, N) == 1
    assert L.spec_early_exit_plan(A, -1, 1.0, E, N) == 1
    assert L.spec_early_exit_plan(A, 3, -0.5, E, N) == 1
    assert L.spec_early_exit_plan(A, 3, float("nan"), E, N) == 1
    assert L.spec_early_exit_plan(A, 3, float("inf"), E, N) == 1
    for bad in (1.5, -0.1, float("inf")):
        b = (ctypes.c_double * 3)(0.5, bad, 0.5)
        assert L.spec_early_exit_plan(ctypes.cast(b, ctypes.c_void_p), 3, 1.0, E, N) == 1
