"""C-ABI checks that need no GPU: the library loads, exports every function
include/specverify.h declares, and rejects bad arguments on the host before
anything is enqueued (status codes only; no compute call runs here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

sv = pytest.importorskip("draft_verification_verify_amd",
                         reason="libspecverify.so not built (run draft_verification_verify_amd/build.py)")
L = sv.lib

FAKE = ctypes.c_void_p(0x100000)       # 16/256-byte aligned, never dereferenced on these paths
FAKE_MIS = ctypes.c_void_p(0x100008)   # misaligned for logits
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+|dcut_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sv.EXPORTED)


def test_status_strings_and_version():
    assert L.spec_verify_abi_version() == 1
    for code, name in sv.STATUS.items():
        assert L.spec_verify_status_string(code).decode() == name
    assert L.spec_verify_status_string(99).decode() == "SV_ERR_UNKNOWN"


def test_timing_arguments_rejected_on_host():
    # argument checks that precede any HIP call
    assert L.spec_verify_timing_begin(-1) == 1
    buf = (ctypes.c_float * 3)()
    assert L.spec_verify_timing_end(buf, 1) == 1       # nothing armed on this thread
    assert L.spec_verify_timing_end(None, -1) == 1


def test_read_ceiling_host_errors():
    assert L.spec_verify_read_ceiling(NULL, 1024, FAKE, NULL) == 1
    assert L.spec_verify_read_ceiling(FAKE, 1024, NULL, NULL) == 1
    assert L.spec_verify_read_ceiling(FAKE, 0, FAKE, NULL) == 1
    assert L.spec_verify_read_ceiling(FAKE, 1000, FAKE, NULL) == 1      # not a multiple of 16
    assert L.spec_verify_read_ceiling(FAKE_MIS, 1024, FAKE, NULL) == 1


def test_workspace_size():
    assert sv.workspace_size(0, 3, 10) == 0
    assert sv.workspace_size(1, -1, 10) == 0
    assert sv.workspace_size(1, 3, 0) == 0
    assert sv.workspace_size(4097, 3, 10) == 0
    assert sv.workspace_size(1, 1025, 10) == 0
    assert sv.workspace_size(1, 3, 2_000_001) == 0
    small = sv.workspace_size(1, 3, 1000)
    big = sv.workspace_size(64, 16, 128000)
    assert 0 < small < big
    assert big % 256 == 0
    assert sv.workspace_size(64, 16, 152064) >= big
    assert big < 64 << 20           # a few MiB, not a copy of the logits


def greedy(target=FAKE, dt=1, tokens=FAKE, depth=NULL, B=4, K=3, V=1000, out=FAKE, num=FAKE,
           ws=FAKE, wsb=None):
    if wsb is None:
        wsb = sv.workspace_size(max(B, 1), max(K, 0), max(V, 1))
    return L.spec_verify_greedy(target, dt, tokens, depth, B, K, V, out, num, ws, wsb, NULL)


def sample(target=FAKE, draft=FAKE, dt=1, tokens=FAKE, depth=NULL, T=FAKE, ua=FAKE, us=FAKE,
           B=4, K=3, V=1000, out=FAKE, num=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = sv.workspace_size(max(B, 1), max(K, 0), max(V, 1))
    return L.spec_verify_sample(target, draft, dt, tokens, depth, T, ua, us, B, K, V, out, num,
                                NULL, NULL, ws, wsb, NULL)


def test_greedy_host_errors():
    assert greedy(target=NULL) == 1
    assert greedy(tokens=NULL) == 1
    assert greedy(out=NULL) == 1
    assert greedy(num=NULL) == 1
    assert greedy(dt=7) == 1
    assert greedy(B=0) == 1
    assert greedy(K=-1) == 1
    assert greedy(V=0) == 1
    assert greedy(B=5000) == 2
    assert greedy(K=2000) == 2
    assert greedy(V=3_000_000) == 2
    assert greedy(target=FAKE_MIS) == 1
    assert greedy(ws=NULL) == 3
    assert greedy(wsb=100) == 3
    assert greedy(ws=ctypes.c_void_p(0x100010)) == 3     # workspace must be 256-byte aligned


def test_sample_host_errors():
    assert sample(target=NULL) == 1
    assert sample(draft=NULL) == 1
    assert sample(T=NULL) == 1
    assert sample(ua=NULL) == 1
    assert sample(us=NULL) == 1
    assert sample(tokens=NULL) == 1
    assert sample(draft=FAKE_MIS) == 1
    assert sample(dt=2) == 1
    assert sample(B=0) == 1
    assert sample(wsb=10) == 3


def test_packed_host_errors():
    wsb = sv.workspace_size(4, 3, 1000)

    def g(target=FAKE, dt=1, tokens=FAKE, offs=FAKE, B=4, K=3, N=8, V=1000, out=FAKE, num=FAKE, ws=FAKE, n=wsb):
        return L.spec_verify_greedy_packed(target, dt, tokens, offs, B, K, N, V, out, num, ws, n, NULL)

    def s(target=FAKE, draft=FAKE, tokens=FAKE, offs=FAKE, T=FAKE, ua=FAKE, us=FAKE, B=4, K=3, N=8, out=FAKE,
          num=FAKE, ws=FAKE, n=wsb):
        return L.spec_verify_sample_packed(target, draft, 1, tokens, offs, T, ua, us, B, K, N, 1000, out, num,
                                           NULL, NULL, ws, n, NULL)

    assert g(offs=NULL) == 1 and g(target=NULL) == 1 and g(tokens=NULL) == 1 and g(out=NULL) == 1
    assert g(num=NULL) == 1 and g(dt=3) == 1 and g(target=FAKE_MIS) == 1
    assert g(N=-1) == 1 and g(N=(1 << 30) + 1) == 2 and g(B=0) == 1 and g(K=2000) == 2
    assert g(ws=NULL) == 3 and g(n=64) == 3
    # no drafted positions: the tokens may be NULL (the workspace check is then reached)
    assert g(tokens=NULL, N=0, ws=NULL) == 3
    assert s(offs=NULL) == 1 and s(target=NULL) == 1 and s(T=NULL) == 1 and s(us=NULL) == 1
    assert s(draft=NULL) == 1 and s(tokens=NULL) == 1 and s(ua=NULL) == 1 and s(draft=FAKE_MIS) == 1
    assert s(N=-5) == 1 and s(N=(1 << 30) + 1) == 2 and s(n=10) == 3
    assert s(draft=NULL, tokens=NULL, ua=NULL, N=0, ws=NULL) == 3


def test_early_exit_host_errors():
    wsb = sv.workspace_size(4, 3, 1000)

    def ends_arg(ends):
        if ends is None:
            return NULL, 0
        arr = (ctypes.c_int32 * max(len(ends), 1))(*ends)
        return ctypes.cast(arr, ctypes.c_void_p), len(ends)

    def g(target=FAKE, dt=1, tokens=FAKE, B=4, K=3, V=1000, ends=(2, 3), out=FAKE, num=FAKE, ws=FAKE, n=wsb):
        ep, ne = ends_arg(ends)
        return L.spec_verify_greedy_early_exit(target, dt, tokens, NULL, B, K, V, ep, ne, out, num, ws, n, NULL)

    def s(target=FAKE, draft=FAKE, T=FAKE, ua=FAKE, us=FAKE, ends=(2, 3), B=4, ws=FAKE, n=wsb):
        ep, ne = ends_arg(ends)
        return L.spec_verify_sample_early_exit(target, draft, 1, FAKE, NULL, T, ua, us, B, 3, 1000, ep, ne,
                                               FAKE, FAKE, NULL, NULL, ws, n, NULL)

    # window ends: null, empty, not increasing, a first end below 1, no end reaching K = 3
    for bad in (None, (), (2, 2, 3), (2, 1, 3), (0, 3), (-1, 3), (1, 2)):
        assert g(ends=bad) == 1, bad
        assert s(ends=bad) == 1, bad
    assert g(target=NULL) == 1 and g(tokens=NULL) == 1 and g(out=NULL) == 1 and g(num=NULL) == 1
    assert g(dt=5) == 1 and g(B=0) == 1 and g(K=-1) == 1 and g(V=0) == 1
    assert g(B=5000) == 2 and g(target=FAKE_MIS) == 1
    # valid ends reach the workspace check (entries after the first end >= K are ignored)
    assert g(ws=NULL) == 3 and g(n=64) == 3 and g(ends=(3, 1, 0), ws=NULL) == 3 and g(ends=(9,), n=64) == 3
    assert s(target=NULL) == 1 and s(draft=NULL) == 1 and s(T=NULL) == 1
    assert s(ua=NULL) == 1 and s(us=NULL) == 1 and s(draft=FAKE_MIS) == 1
    assert s(B=0) == 1 and s(n=10) == 3


def test_confidence_and_dcut_host_errors():
    wsb = sv.workspace_size(4, 3, 1000)
    assert L.spec_draft_confidence(NULL, 1, NULL, 4, 3, 1000, FAKE, FAKE, wsb, NULL) == 1
    assert L.spec_draft_confidence(FAKE, 1, NULL, 4, 3, 1000, NULL, FAKE, wsb, NULL) == 1
    assert L.spec_draft_confidence(FAKE, 1, NULL, 4, 3, 1000, FAKE, FAKE, 16, NULL) == 3
    assert L.spec_draft_confidence(FAKE, 1, NULL, 0, 3, 1000, FAKE, FAKE, wsb, NULL) == 1
    assert L.dcut_allocate(FAKE, NULL, 4, 3, 3, FAKE, NULL) == 4         # budget < B
    assert L.dcut_allocate(FAKE, NULL, 0, 3, 3, FAKE, NULL) == 1
    assert L.dcut_allocate(NULL, NULL, 4, 3, 8, FAKE, NULL) == 1
    assert L.dcut_allocate(FAKE, NULL, 4, 3, 8, NULL, NULL) == 1
    assert L.dcut_allocate(FAKE, NULL, 4096, 16, 9000, FAKE, NULL) == 2  # B*K > 32768


def test_reuse_entry_points_host_errors():
    wsb = sv.workspace_size(4, 3, 1000)
    stats, stats_mis = FAKE, ctypes.c_void_p(0x100008)
    # spec_draft_confidence_stats: stats required and 16-byte aligned, conf optional
    cs = L.spec_draft_confidence_stats
    assert cs(NULL, 1, NULL, 4, 3, 1000, FAKE, stats, FAKE, wsb, NULL) == 1
    assert cs(FAKE, 1, NULL, 4, 3, 1000, FAKE, NULL, FAKE, wsb, NULL) == 1
    assert cs(FAKE, 1, NULL, 4, 3, 1000, FAKE, stats_mis, FAKE, wsb, NULL) == 1
    assert cs(FAKE, 1, NULL, 4, 3, 1000, NULL, stats, FAKE, 16, NULL) == 3
    assert cs(FAKE, 9, NULL, 4, 3, 1000, NULL, stats, FAKE, wsb, NULL) == 1
    # spec_draft_confidence_stats_t: the temperatures are required too
    ct = L.spec_draft_confidence_stats_t
    assert ct(FAKE, 1, NULL, NULL, 4, 3, 1000, FAKE, stats, FAKE, wsb, NULL) == 1
    assert ct(NULL, 1, NULL, FAKE, 4, 3, 1000, FAKE, stats, FAKE, wsb, NULL) == 1
    assert ct(FAKE, 1, NULL, FAKE, 4, 3, 1000, FAKE, NULL, FAKE, wsb, NULL) == 1
    assert ct(FAKE, 1, NULL, FAKE, 4, 3, 1000, FAKE, stats_mis, FAKE, wsb, NULL) == 1
    assert ct(FAKE, 1, NULL, FAKE, 4, 3, 1000, NULL, stats, FAKE, 16, NULL) == 3
    assert ct(FAKE, 1, NULL, FAKE, 0, 3, 1000, NULL, stats, FAKE, wsb, NULL) == 1
    # spec_verify_sample_reuse: the statistics are required when K > 0
    def reuse(draft_stats=stats, **kw):
        a = dict(target=FAKE, draft=FAKE, dt=1, tokens=FAKE, depth=NULL, T=FAKE, ua=FAKE, us=FAKE,
                 B=4, K=3, V=1000, out=FAKE, num=FAKE, ws=FAKE, wsb=wsb)
        a.update(kw)
        return L.spec_verify_sample_reuse(a["target"], a["draft"], a["dt"], a["tokens"], a["depth"], a["T"],
                                          a["ua"], a["us"], draft_stats, a["B"], a["K"], a["V"], a["out"],
                                          a["num"], NULL, NULL, a["ws"], a["wsb"], NULL)
    assert reuse(draft_stats=NULL) == 1
    assert reuse(draft_stats=stats_mis) == 1
    assert reuse(target=NULL) == 1
    assert reuse(draft=NULL) == 1
    assert reuse(us=NULL) == 1
    assert reuse(wsb=10) == 3


def test_dcut_cost_host_errors():
    f = L.dcut_allocate_cost
    dbl = ctypes.c_double

    def tab(*v):
        return ctypes.cast((dbl * len(v))(*v), ctypes.c_void_p)
    td, tc = tab(1.0, 2.0, 4.0), tab(1.0, 1.2, 1.5)
    assert f(NULL, NULL, 4, 3, td, tc, 3, 10.0, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, td, tc, 3, 10.0, NULL, NULL) == 1
    assert f(FAKE, NULL, 0, 3, td, tc, 3, 10.0, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, NULL, tc, 3, 10.0, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, td, tc, 0, 10.0, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, td, tc, 33, 10.0, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, td, tc, 3, -1.0, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, td, tc, 3, float("nan"), FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, td, tc, 3, float("inf"), FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, tab(1.0, 1.0, 4.0), tc, 3, 10.0, FAKE, NULL) == 1    # depths not increasing
    assert f(FAKE, NULL, 4, 3, td, tab(1.0, 0.0, 1.5), 3, 10.0, FAKE, NULL) == 1    # a cost not > 0
    assert f(FAKE, NULL, 5000, 3, td, tc, 3, 10.0, FAKE, NULL) == 2


def test_accept_stats_host_errors():
    f = L.spec_accept_stats_update
    assert f(NULL, NULL, 4, 3, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, NULL, NULL) == 1
    assert f(FAKE, NULL, 0, 3, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, -1, FAKE, NULL) == 1
    assert f(FAKE, NULL, 4, 3, ctypes.c_void_p(0x100004), NULL) == 1   # counters 8-byte aligned
    assert f(FAKE, NULL, 5000, 3, FAKE, NULL) == 2


def test_binding_shares_torch_hip_runtime():
    # exactly one HIP runtime in the process, the one torch loaded
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_noalloc_host_errors():
    # argument and size checks that precede any HIP call
    def call(B=4, K=3, V=1000, target=FAKE, draft=FAKE, temp=FAKE, us=FAKE, out=FAKE, num=FAKE, dt=1):
        return L.spec_verify_sample_noalloc(target, draft, dt, FAKE, NULL, temp, FAKE, us, B, K, V, out, num,
                                            NULL, NULL, NULL)
    assert call(target=NULL) == 1 and call(temp=NULL) == 1 and call(out=NULL) == 1 and call(num=NULL) == 1
    assert call(draft=NULL) == 1 and call(dt=7) == 1 and call(target=FAKE_MIS) == 1
    assert call(B=0) == 1 and call(B=4097) == 2
    # the workspace of B=256, K=64, V=128000 exceeds the 8 MiB static array
    assert sv.workspace_size(256, 64, 128000) > sv.NOALLOC_SCRATCH_BYTES
    assert call(B=256, K=64, V=128000) == 2
    assert "static array" in L.spec_verify_last_error().decode()
    # the headline shapes fit
    assert sv.workspace_size(64, 16, 152064) <= sv.NOALLOC_SCRATCH_BYTES
