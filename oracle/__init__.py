"""ctypes front end of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module; the product path (the HIP library and
its binding) never does.  The oracle is plain single-threaded C in double
precision; this module only marshals numpy arrays into it.

Storage convention for logits: bf16 tensors are passed as ``numpy.uint16``
(the raw upper halves of IEEE binary32 words), fp32 as ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of oracle.c (the mutation test
# builds deliberately broken copies to show the pins catch them).
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")

DT_F32 = 0
DT_BF16 = 1


def compile_to(src: str, out: str) -> str:
    """gcc build of an oracle source (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
        "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into oracle/liboracle.so."""
    if _LIB_OVERRIDE:
        return _LIB_OVERRIDE
    if force or not os.path.exists(_LIB):
        compile_to(_SRC, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            L = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_argmax.argtypes = [vp, ctypes.c_int, i64]
        L.oracle_argmax.restype = i64
        L.oracle_softmax.argtypes = [vp, ctypes.c_int, i64, dbl, vp, vp, vp]
        L.oracle_softmax.restype = ctypes.c_int
        L.oracle_inverse_cdf.argtypes = [vp, i64, dbl]
        L.oracle_inverse_cdf.restype = i64
        L.oracle_residual.argtypes = [vp, vp, ctypes.c_int, i64, dbl, vp]
        L.oracle_residual.restype = ctypes.c_int
        L.oracle_verify_greedy.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i64, vp, vp]
        L.oracle_verify_greedy.restype = ctypes.c_int
        L.oracle_verify_sample.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                           i32, i32, i64, vp, vp, vp, vp, vp]
        L.oracle_verify_sample.restype = ctypes.c_int
        L.oracle_verify_early_exit.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp,
                                               i32, i32, i64, vp, vp, vp, vp]
        L.oracle_verify_early_exit.restype = ctypes.c_int
        L.oracle_draft_confidence.argtypes = [vp, ctypes.c_int, vp, i32, i32, i64, vp]
        L.oracle_draft_confidence.restype = ctypes.c_int
        L.oracle_dcut_allocate.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_dcut_allocate.restype = ctypes.c_int
        L.oracle_accept_stats.argtypes = [vp, vp, i32, i32, vp]
        L.oracle_accept_stats.restype = ctypes.c_int
        L.oracle_dcut_cost.argtypes = [vp, vp, i32, dbl]
        L.oracle_dcut_cost.restype = dbl
        L.oracle_dcut_allocate_cost.argtypes = [vp, vp, i32, i32, vp, vp, i32, dbl, vp]
        L.oracle_dcut_allocate_cost.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    raise TypeError(f"logits must be uint16 (bf16 bits) or float32, got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def argmax(row: np.ndarray) -> int:
    row = _c(row)
    return int(lib().oracle_argmax(_ptr(row), _dt(row), row.size))


def softmax(row: np.ndarray, T: float = 1.0):
    """Returns (P as float64 array, M, S); raises ValueError on a bad row."""
    row = _c(row)
    p = np.empty(row.size, np.float64)
    M = ctypes.c_double()
    S = ctypes.c_double()
    rc = lib().oracle_softmax(_ptr(row), _dt(row), row.size, float(T), _ptr(p),
                              ctypes.byref(M), ctypes.byref(S))
    if rc != 0:
        raise ValueError(f"bad row (code {rc})")
    return p, M.value, S.value


def inverse_cdf(r: np.ndarray, u: float) -> int:
    r = _c(r, np.float64)
    return int(lib().oracle_inverse_cdf(_ptr(r), r.size, float(u)))


def residual(trow: np.ndarray, drow, T: float):
    """Returns (r as float64 array, fell_back: bool)."""
    trow = _c(trow)
    drow = _c(drow)
    r = np.empty(trow.size, np.float64)
    rc = lib().oracle_residual(_ptr(trow), _ptr(drow), _dt(trow), trow.size, float(T), _ptr(r))
    if rc in (1, 2):
        raise ValueError(f"bad row (code {rc})")
    return r, rc == 3


def verify_greedy(target, tokens, depth=None):
    """target [B,K+1,V] (uint16 bf16 bits or float32); returns (out[B,K+1], n[B])."""
    target = _c(target)
    B, K1, V = target.shape
    K = K1 - 1
    tokens = _c(tokens, np.int32).reshape(B, K)
    depth = _c(depth, np.int32)
    out = np.empty((B, K + 1), np.int32)
    n = np.empty(B, np.int32)
    lib().oracle_verify_greedy(_ptr(target), _dt(target), _ptr(tokens), _ptr(depth),
                               B, K, V, _ptr(out), _ptr(n))
    return out, n


def verify_sample(target, draft, tokens, temperature, u_accept, u_sample, depth=None):
    """Returns dict with out, n, p_draft, q_draft (float32 [B,K]) and ratio (float64 [B,K])."""
    target = _c(target)
    B, K1, V = target.shape
    K = K1 - 1
    draft = _c(draft)
    if draft.dtype != target.dtype or draft.shape != (B, K, V):
        raise ValueError("draft must match target dtype and have shape [B,K,V]")
    tokens = _c(tokens, np.int32).reshape(B, K)
    temperature = _c(temperature, np.float32).reshape(B)
    u_accept = _c(u_accept, np.float32).reshape(B, K)
    u_sample = _c(u_sample, np.float32).reshape(B)
    depth = _c(depth, np.int32)
    out = np.empty((B, K + 1), np.int32)
    n = np.empty(B, np.int32)
    p = np.empty((B, K), np.float32)
    q = np.empty((B, K), np.float32)
    ratio = np.empty((B, K), np.float64)
    lib().oracle_verify_sample(_ptr(target), _ptr(draft), _dt(target), _ptr(tokens), _ptr(depth),
                               _ptr(temperature), _ptr(u_accept), _ptr(u_sample), B, K, V,
                               _ptr(out), _ptr(n), _ptr(p), _ptr(q), _ptr(ratio))
    return {"out": out, "n": n, "p_draft": p, "q_draft": q, "ratio": ratio}


def verify_early_exit(target, tokens, draft=None, temperature=None, u_accept=None, u_sample=None,
                      depth=None):
    """Sequential (early-exit) verification: positions in order, stop at the
    first rejection, nothing after it read.  temperature None means every
    request uses the greedy rule (draft and uniforms may then be None).
    Returns dict with out, n, p_draft, q_draft (float32 [B,K])."""
    target = _c(target)
    B, K1, V = target.shape
    K = K1 - 1
    tokens = _c(tokens, np.int32).reshape(B, K)
    if temperature is not None:
        draft = _c(draft)
        if draft.dtype != target.dtype or draft.shape != (B, K, V):
            raise ValueError("draft must match target dtype and have shape [B,K,V]")
        temperature = _c(temperature, np.float32).reshape(B)
        u_accept = _c(u_accept, np.float32).reshape(B, K)
        u_sample = _c(u_sample, np.float32).reshape(B)
    else:
        draft = u_accept = u_sample = None
    depth = _c(depth, np.int32)
    out = np.empty((B, K + 1), np.int32)
    n = np.empty(B, np.int32)
    p = np.empty((B, K), np.float32)
    q = np.empty((B, K), np.float32)
    lib().oracle_verify_early_exit(_ptr(target), _ptr(draft), _dt(target), _ptr(tokens), _ptr(depth),
                                   _ptr(temperature), _ptr(u_accept), _ptr(u_sample), B, K, V,
                                   _ptr(out), _ptr(n), _ptr(p), _ptr(q))
    return {"out": out, "n": n, "p_draft": p, "q_draft": q}


def draft_confidence(draft, max_depth=None):
    draft = _c(draft)
    B, K, V = draft.shape
    max_depth = _c(max_depth, np.int32)
    conf = np.empty((B, K), np.float32)
    lib().oracle_draft_confidence(_ptr(draft), _dt(draft), _ptr(max_depth), B, K, V, _ptr(conf))
    return conf


def dcut_allocate(conf, budget: int, max_depth=None):
    """Returns depth[B] (int32); raises ValueError for B<1 or budget < B."""
    conf = _c(conf, np.float32)
    B, K = conf.shape
    max_depth = _c(max_depth, np.int32)
    depth = np.empty(B, np.int32)
    rc = lib().oracle_dcut_allocate(_ptr(conf), _ptr(max_depth), B, K, int(budget), _ptr(depth))
    if rc != 0:
        raise ValueError(f"dcut_allocate rejected its arguments (code {rc})")
    return depth


def accept_stats(num_accepted, K: int, depth=None, counters=None):
    """Adds one call's acceptance statistics into counters[2K + 4] (uint64):
    reached[0:K], accepted[K:2K], then requests, bad, sum n, sum (n + 1)."""
    num_accepted = _c(num_accepted, np.int32)
    B = num_accepted.shape[0]
    depth = _c(depth, np.int32)
    if counters is None:
        counters = np.zeros(2 * K + 4, np.uint64)
    assert counters.dtype == np.uint64 and counters.shape == (2 * K + 4,)
    rc = lib().oracle_accept_stats(_ptr(num_accepted), _ptr(depth), B, K, _ptr(counters))
    if rc != 0:
        raise ValueError(f"accept_stats rejected its arguments (code {rc})")
    return counters


# the latency table printed with the pages' cost-aware D-cut sketch (depth: relative cost)
DEFAULT_COST_TABLE = ((1.0, 1.0), (2.0, 1.2), (4.0, 1.5), (8.0, 2.0), (16.0, 3.0))


def _table(table):
    t = np.ascontiguousarray([p[0] for p in table], np.float64)
    c = np.ascontiguousarray([p[1] for p in table], np.float64)
    return t, c


def dcut_cost(d: float, table=DEFAULT_COST_TABLE) -> float:
    t, c = _table(table)
    return float(lib().oracle_dcut_cost(_ptr(t), _ptr(c), len(t), float(d)))


def dcut_allocate_cost(conf, max_verify: float, max_depth=None, table=DEFAULT_COST_TABLE):
    """Cost-aware D-cut: depth[B] (int32), 0 for requests not admitted."""
    conf = _c(conf, np.float32)
    B, K = conf.shape
    max_depth = _c(max_depth, np.int32)
    t, c = _table(table)
    depth = np.empty(B, np.int32)
    rc = lib().oracle_dcut_allocate_cost(_ptr(conf), _ptr(max_depth), B, K, _ptr(t), _ptr(c), len(t),
                                         float(max_verify), _ptr(depth))
    if rc != 0:
        raise ValueError(f"dcut_allocate_cost rejected its arguments (code {rc})")
    return depth

