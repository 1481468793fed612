"""Python binding of libspecverify (batched draft verification on MI355X).

Argument marshalling only: every step of verification runs in the HIP
kernels of ``libspecverify.so`` (built from ``csrc/specverify.hip`` by
``build.py``).  torch supplies device memory and the stream; tensors must be
contiguous and on the current GPU.  If the shared library is missing this
module raises at import time -- there is no fallback path.

Calls mirror the C ABI in ``include/specverify.h``:

    verify_greedy(target, tokens, depth=None)            -> (out_tokens, num_accepted)
    verify_sample(target, draft, tokens, temperature,
                  u_accept, u_sample, depth=None)        -> (out_tokens, num_accepted, p_draft, q_draft)
    verify_greedy_packed(target, tokens, offsets, K_max) -> (out_tokens, num_accepted)
    verify_sample_packed(target, draft, tokens, offsets, temperature,
                         u_accept, u_sample, K_max)      -> (out_tokens, num_accepted, p_draft, q_draft)
    draft_confidence(draft, max_depth=None)              -> conf
    dcut_allocate(conf, budget, max_depth=None)          -> depth
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
STATUS = {0: "SV_OK", 1: "SV_ERR_INVALID_ARG", 2: "SV_ERR_UNSUPPORTED", 3: "SV_ERR_WORKSPACE",
          4: "SV_ERR_BUDGET", 5: "SV_ERR_BAD_INPUT", 6: "SV_ERR_HIP"}


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}" + (f": {detail}" if detail else ""))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python draft_verification_verify_amd/build.py`")
    # torch ships its own HIP runtime (loaded by its unversioned file name).
    # Import it first so that libspecverify binds to that same runtime via its
    # soname; loading ours first would put two HIP runtimes in the process,
    # and device memory from one is unusable by kernels launched on the other.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.spec_verify_abi_version.restype = i32
    L.spec_verify_abi_version.argtypes = []
    L.spec_verify_status_string.restype = ctypes.c_char_p
    L.spec_verify_status_string.argtypes = [ctypes.c_int]
    L.spec_verify_last_error.restype = ctypes.c_char_p
    L.spec_verify_last_error.argtypes = []
    L.spec_verify_workspace_size.restype = sz
    L.spec_verify_workspace_size.argtypes = [i32, i32, i32]
    L.spec_verify_greedy.restype = ctypes.c_int
    L.spec_verify_greedy.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.spec_verify_sample.restype = ctypes.c_int
    L.spec_verify_sample.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32,
                                     vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_greedy_packed.restype = ctypes.c_int
    L.spec_verify_greedy_packed.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    L.spec_verify_sample_packed.restype = ctypes.c_int
    L.spec_verify_sample_packed.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                            vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_sample_noalloc.restype = ctypes.c_int
    L.spec_verify_sample_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32,
                                             vp, vp, vp, vp, vp]
    L.spec_verify_greedy_early_exit.restype = ctypes.c_int
    L.spec_verify_greedy_early_exit.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, sz,
                                                vp]
    L.spec_verify_sample_early_exit.restype = ctypes.c_int
    L.spec_verify_sample_early_exit.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, vp, i32,
                                                vp, vp, vp, vp, vp, sz, vp]
    L.spec_draft_confidence.restype = ctypes.c_int
    L.spec_draft_confidence.argtypes = [vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, sz, vp]
    L.spec_draft_confidence_stats_t.restype = ctypes.c_int
    L.spec_draft_confidence_stats_t.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.spec_draft_confidence_stats.restype = ctypes.c_int
    L.spec_draft_confidence_stats.argtypes = [vp, ctypes.c_int, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.spec_verify_sample_reuse.restype = ctypes.c_int
    L.spec_verify_sample_reuse.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                           vp, vp, vp, vp, vp, sz, vp]
    L.spec_accept_stats_summary.restype = ctypes.c_int
    L.spec_accept_stats_summary.argtypes = [vp, i32, vp, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double)]
    L.dcut_allocate_cost.restype = ctypes.c_int
    L.dcut_allocate_cost.argtypes = [vp, vp, i32, i32, vp, vp, i32, ctypes.c_double, vp, vp]
    L.spec_accept_stats_update.restype = ctypes.c_int
    L.spec_accept_stats_update.argtypes = [vp, vp, i32, i32, vp, vp]
    L.dcut_allocate.restype = ctypes.c_int
    L.dcut_allocate.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.spec_early_exit_plan.restype = ctypes.c_int
    L.spec_early_exit_plan.argtypes = [vp, i32, ctypes.c_double, vp, vp]
    L.spec_verify_read_ceiling.restype = ctypes.c_int
    L.spec_verify_read_ceiling.argtypes = [vp, sz, vp, vp]
    L.spec_verify_timing_begin.restype = ctypes.c_int
    L.spec_verify_timing_begin.argtypes = [i32]
    L.spec_verify_timing_end.restype = ctypes.c_int
    L.spec_verify_timing_end.argtypes = [ctypes.POINTER(ctypes.c_float), i32]
    if L.spec_verify_abi_version() != 1:
        raise ImportError("libspecverify ABI version mismatch")
    return L


lib = _load()

EXPORTED = ("spec_verify_abi_version", "spec_verify_status_string", "spec_verify_last_error",
            "spec_verify_workspace_size", "spec_verify_timing_begin", "spec_verify_timing_end",
            "spec_verify_greedy", "spec_verify_sample", "spec_draft_confidence", "dcut_allocate",
            "spec_draft_confidence_stats", "spec_verify_sample_reuse", "spec_accept_stats_update",
            "dcut_allocate_cost", "spec_verify_greedy_early_exit", "spec_verify_sample_early_exit",
            "spec_verify_read_ceiling", "spec_early_exit_plan", "spec_verify_sample_noalloc",
            "spec_accept_stats_summary", "spec_verify_greedy_packed", "spec_verify_sample_packed",
            "spec_draft_confidence_stats_t")

# Bytes of the static scratch array behind spec_verify_sample_noalloc.
NOALLOC_SCRATCH_BYTES = 8 << 20


def workspace_size(B: int, K: int, V: int) -> int:
    return int(lib.spec_verify_workspace_size(B, K, V))


def read_ceiling(buf, sink=None, stream=None):
    """Benchmark instrumentation: one plain read of every byte of ``buf`` (a
    contiguous CUDA tensor) with the row-statistics kernel's load width."""
    torch = _torch()
    _validate((buf, "buf", None, None), (sink, "sink", torch.int32, (1,)))
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    st = lib.spec_verify_read_ceiling(_ptr(buf), nbytes, _ptr(sink), _stream(stream))
    _raise("spec_verify_read_ceiling", st)
    return sink


def timing_begin(n: int) -> None:
    """Arm per-kernel event timing for this thread's next ``n`` verification calls."""
    st = lib.spec_verify_timing_begin(int(n))
    if st:
        _raise("spec_verify_timing_begin", st)


def timing_end(n: int):
    """Wait for the armed calls and return an (n, 3) list of stage milliseconds:
    row statistics, finish (merge, accept scan, sampler sums), draw."""
    buf = (ctypes.c_float * (3 * max(int(n), 1)))()
    st = lib.spec_verify_timing_end(buf, int(n))
    if st:
        _raise("spec_verify_timing_end", st)
    return [[buf[3 * i + s] for s in range(3)] for i in range(int(n))]


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _shape3(t, name):
    """(B, rows, V) of a 3-D logits tensor."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D [B, rows, V], got shape {tuple(t.shape)}")
    return tuple(int(x) for x in t.shape)


def _validate(*specs, device=None):
    """Checks every tensor argument of a call before any pointer is taken.

    specs: (tensor or None, name, dtype or None, shape or None).  First the
    dtype, shape and contiguity of every argument, then that every one is a
    GPU tensor on ``device`` (default: the first argument's).  A wrong-sized
    output or a host tensor would otherwise become an out-of-bounds or
    host-address device write."""
    torch = _torch()
    present = [sp for sp in specs if sp[0] is not None]
    for t, name, dtype, shape in present:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if device is None and present:
        device = present[0][0].device
    for t, name, _, _ in present:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}; the call's tensors are on {device}")


class Workspace:
    """A device buffer reused across calls on one device (grown on demand).

    Each call writes every part of the workspace it later reads, so contents
    never matter.  Calls that share a workspace must be ordered on one
    stream."""

    def __init__(self):
        self._buf = {}
        self._lock = threading.Lock()

    def get(self, device, nbytes: int):
        torch = _torch()
        key = torch.device(device).index if torch.device(device).index is not None else torch.cuda.current_device()
        with self._lock:
            buf = self._buf.get(key)
            if buf is None or buf.numel() < nbytes:
                buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=torch.device("cuda", key))
                self._buf[key] = buf
            return buf


_default_ws = Workspace()


def _ws(device, B, K, V, workspace):
    """(buffer, byte count) of the workspace: the caller's (a contiguous GPU
    tensor on the call's device, any dtype) or the shared default."""
    n = workspace_size(B, K, V)
    if n == 0:
        raise SpecVerifyError("spec_verify_workspace_size", 2)
    if workspace is None:
        return _default_ws.get(device, n), n
    _validate((workspace, "workspace", None, None), device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _raise(fn, st):
    if st != 0:
        named = st in (5, 6) or (st == 2 and fn == "spec_verify_sample_noalloc")
        detail = lib.spec_verify_last_error().decode() if named else ""
        raise SpecVerifyError(fn, st, detail)


def _sample_specs(target, draft, tokens, temperature, u_accept, u_sample, depth, B, K, V):
    torch = _torch()
    return [(target, "target", None, None), (draft, "draft", target.dtype, (B, K, V)),
            (tokens, "tokens", torch.int32, (B, K)), (temperature, "temperature", torch.float32, (B,)),
            (u_accept, "u_accept", torch.float32, (B, K)), (u_sample, "u_sample", torch.float32, (B,)),
            (depth, "depth", torch.int32, (B,))]


def _out_specs(B, K, out_tokens, num_accepted, p_draft=None, q_draft=None):
    torch = _torch()
    return [(out_tokens, "out_tokens", torch.int32, (B, K + 1)), (num_accepted, "num_accepted", torch.int32, (B,)),
            (p_draft, "p_draft", torch.float32, (B, K)), (q_draft, "q_draft", torch.float32, (B, K))]


def _new_outputs(dev, B, K, out_tokens, num_accepted, p_draft=None, q_draft=None, want_probs=False):
    torch = _torch()
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if want_probs and p_draft is None:
        p_draft = torch.empty((B, K), dtype=torch.float32, device=dev)
    if want_probs and q_draft is None:
        q_draft = torch.empty((B, K), dtype=torch.float32, device=dev)
    return out_tokens, num_accepted, p_draft, q_draft


def verify_greedy(target, tokens, depth=None, *, out_tokens=None, num_accepted=None,
                  workspace=None, stream=None):
    """Greedy (T=0) verification.  target [B,K+1,V] bf16/fp32, tokens [B,K] int32."""
    torch = _torch()
    B, K1, V = _shape3(target, "target")
    K = K1 - 1
    dt = _dtype_code(target)
    _validate((target, "target", None, None), (tokens, "tokens", torch.int32, (B, K)),
              (depth, "depth", torch.int32, (B,)), *_out_specs(B, K, out_tokens, num_accepted))
    out_tokens, num_accepted, _, _ = _new_outputs(target.device, B, K, out_tokens, num_accepted)
    ws, nbytes = _ws(target.device, B, K, V, workspace)
    st = lib.spec_verify_greedy(_ptr(target), dt, _ptr(tokens), _ptr(depth), B, K, V,
                                _ptr(out_tokens), _ptr(num_accepted), _ptr(ws), nbytes, _stream(stream))
    _raise("spec_verify_greedy", st)
    return out_tokens, num_accepted


def verify_sample(target, draft, tokens, temperature, u_accept, u_sample, depth=None, *,
                  out_tokens=None, num_accepted=None, p_draft=None, q_draft=None,
                  want_probs: bool = True, workspace=None, stream=None):
    """Rejection-sampling verification.  Returns (out_tokens, num_accepted, p_draft, q_draft)."""
    B, K1, V = _shape3(target, "target")
    K = K1 - 1
    dt = _dtype_code(target)
    _validate(*_sample_specs(target, draft, tokens, temperature, u_accept, u_sample, depth, B, K, V),
              *_out_specs(B, K, out_tokens, num_accepted, p_draft, q_draft))
    out_tokens, num_accepted, p_draft, q_draft = _new_outputs(target.device, B, K, out_tokens, num_accepted,
                                                              p_draft, q_draft, want_probs)
    ws, nbytes = _ws(target.device, B, K, V, workspace)
    st = lib.spec_verify_sample(_ptr(target), _ptr(draft), dt, _ptr(tokens), _ptr(depth),
                                _ptr(temperature), _ptr(u_accept), _ptr(u_sample), B, K, V,
                                _ptr(out_tokens), _ptr(num_accepted), _ptr(p_draft), _ptr(q_draft),
                                _ptr(ws), nbytes, _stream(stream))
    _raise("spec_verify_sample", st)
    return out_tokens, num_accepted, p_draft, q_draft


def _packed_shape(target, tokens, offsets):
    """(B, N, V) of a packed call: offsets [B + 1], tokens [N], target [N + B, V]."""
    torch = _torch()
    for t, name in ((target, "target"), (tokens, "tokens"), (offsets, "offsets")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if offsets.dim() != 1 or offsets.numel() < 2:
        raise ValueError(f"offsets must be 1-D [B + 1] with B >= 1, got shape {tuple(offsets.shape)}")
    if tokens.dim() != 1:
        raise ValueError(f"tokens must be 1-D [N], got shape {tuple(tokens.shape)}")
    B, N = offsets.numel() - 1, tokens.numel()
    if target.dim() != 2 or target.shape[0] != N + B:
        raise ValueError(f"target must be 2-D [N + B, V] = [{N + B}, V], got shape {tuple(target.shape)}")
    return B, N, int(target.shape[1])


def _packed_outputs(dev, B, N, out_tokens, num_accepted, p_draft=None, q_draft=None, want_probs=False):
    torch = _torch()
    if out_tokens is None:
        out_tokens = torch.empty((N + B,), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if want_probs and p_draft is None:
        p_draft = torch.empty((N,), dtype=torch.float32, device=dev)
    if want_probs and q_draft is None:
        q_draft = torch.empty((N,), dtype=torch.float32, device=dev)
    return out_tokens, num_accepted, p_draft, q_draft


def verify_greedy_packed(target, tokens, offsets, K_max: int, *, out_tokens=None, num_accepted=None,
                         workspace=None, stream=None):
    """Greedy verification, packed layout: request b's drafted positions are
    offsets[b] .. offsets[b+1]-1 of tokens [N]; its target rows start at row
    offsets[b] + b of target [N + B, V].  Returns (out_tokens [N + B],
    num_accepted [B])."""
    torch = _torch()
    B, N, V = _packed_shape(target, tokens, offsets)
    dt = _dtype_code(target)
    _validate((target, "target", None, None), (tokens, "tokens", torch.int32, (N,)),
              (offsets, "offsets", torch.int32, (B + 1,)),
              (out_tokens, "out_tokens", torch.int32, (N + B,)), (num_accepted, "num_accepted", torch.int32, (B,)))
    out_tokens, num_accepted, _, _ = _packed_outputs(target.device, B, N, out_tokens, num_accepted)
    ws, nbytes = _ws(target.device, B, int(K_max), V, workspace)
    st = lib.spec_verify_greedy_packed(_ptr(target), dt, _ptr(tokens) if N else None, _ptr(offsets), B,
                                       int(K_max), N, V, _ptr(out_tokens), _ptr(num_accepted), _ptr(ws),
                                       nbytes, _stream(stream))
    _raise("spec_verify_greedy_packed", st)
    return out_tokens, num_accepted


def verify_sample_packed(target, draft, tokens, offsets, temperature, u_accept, u_sample, K_max: int, *,
                         out_tokens=None, num_accepted=None, p_draft=None, q_draft=None,
                         want_probs: bool = True, workspace=None, stream=None):
    """Rejection-sampling verification, packed layout: draft [N, V],
    tokens / u_accept [N], target [N + B, V], offsets [B + 1] (see
    verify_greedy_packed); temperature and u_sample [B].  Returns
    (out_tokens [N + B], num_accepted [B], p_draft [N], q_draft [N])."""
    torch = _torch()
    B, N, V = _packed_shape(target, tokens, offsets)
    dt = _dtype_code(target)
    _validate((target, "target", None, None), (draft, "draft", target.dtype, (N, V)),
              (tokens, "tokens", torch.int32, (N,)), (offsets, "offsets", torch.int32, (B + 1,)),
              (temperature, "temperature", torch.float32, (B,)), (u_accept, "u_accept", torch.float32, (N,)),
              (u_sample, "u_sample", torch.float32, (B,)),
              (out_tokens, "out_tokens", torch.int32, (N + B,)), (num_accepted, "num_accepted", torch.int32, (B,)),
              (p_draft, "p_draft", torch.float32, (N,)), (q_draft, "q_draft", torch.float32, (N,)))
    out_tokens, num_accepted, p_draft, q_draft = _packed_outputs(target.device, B, N, out_tokens, num_accepted,
                                                                 p_draft, q_draft, want_probs)
    ws, nbytes = _ws(target.device, B, int(K_max), V, workspace)
    nz = (lambda t: _ptr(t) if N else None)
    st = lib.spec_verify_sample_packed(_ptr(target), nz(draft), dt, nz(tokens), _ptr(offsets),
                                       _ptr(temperature), nz(u_accept), _ptr(u_sample), B, int(K_max), N, V,
                                       _ptr(out_tokens), _ptr(num_accepted), nz(p_draft), nz(q_draft),
                                       _ptr(ws), nbytes, _stream(stream))
    _raise("spec_verify_sample_packed", st)
    return out_tokens, num_accepted, p_draft, q_draft


def verify_sample_noalloc(target, draft, tokens, temperature, u_accept, u_sample, depth=None, *,
                          out_tokens, num_accepted, p_draft=None, q_draft=None, stream=None):
    """verify_sample without a workspace: the library's static device scratch
    serves instead, and the call allocates nothing (the caller passes every
    output).  Calls that may overlap on one GPU must be serialised."""
    B, K1, V = _shape3(target, "target")
    K = K1 - 1
    dt = _dtype_code(target)
    if out_tokens is None or num_accepted is None:
        raise ValueError("verify_sample_noalloc allocates nothing: pass out_tokens and num_accepted")
    _validate(*_sample_specs(target, draft, tokens, temperature, u_accept, u_sample, depth, B, K, V),
              *_out_specs(B, K, out_tokens, num_accepted, p_draft, q_draft))
    st = lib.spec_verify_sample_noalloc(_ptr(target), _ptr(draft), dt, _ptr(tokens), _ptr(depth),
                                        _ptr(temperature), _ptr(u_accept), _ptr(u_sample), B, K, V,
                                        _ptr(out_tokens), _ptr(num_accepted), _ptr(p_draft), _ptr(q_draft),
                                        _stream(stream))
    _raise("spec_verify_sample_noalloc", st)
    return out_tokens, num_accepted, p_draft, q_draft


def window_ends(K: int, window=None, ends=None):
    """Window ends for the early-exit calls: ``ends`` as given, else fixed
    windows of ``window`` positions (W, 2W, ... up to K), else a first
    window of about K/4 positions and one window for the rest."""
    if ends is not None:
        return [int(e) for e in ends]
    if window is not None:
        W = int(window)
        if W < 1:
            raise ValueError("window must be >= 1")
        return [W * i for i in range(1, max(1, -(-K // W)) + 1)]
    first = max(1, (K + 3) // 4)
    return [first, K] if first < K else [max(K, 1)]


def early_exit_plan(alpha, window_cost: float = 2.5):
    """Window ends minimising the expected cost for per-position acceptance
    ``alpha`` (a sequence of K rates in [0, 1]; NaN, a position no request
    reached, counts as 0).  ``window_cost``: a window's fixed latency in
    units of streaming one position of the batch."""
    a = [float(x) for x in alpha]
    K = len(a)
    arr = (ctypes.c_double * max(K, 1))(*a)
    ends = (ctypes.c_int32 * max(K, 1))()
    n = ctypes.c_int32(0)
    st = lib.spec_early_exit_plan(ctypes.cast(arr, ctypes.c_void_p), K, float(window_cost),
                                  ctypes.cast(ends, ctypes.c_void_p), ctypes.cast(ctypes.pointer(n), ctypes.c_void_p))
    _raise("spec_early_exit_plan", st)
    return [int(ends[i]) for i in range(n.value)]


def _ends_arg(ends):
    arr = (ctypes.c_int32 * len(ends))(*ends)
    return ctypes.cast(arr, ctypes.c_void_p), len(ends), arr


def verify_greedy_early_exit(target, tokens, depth=None, *, window=None, ends=None, out_tokens=None,
                             num_accepted=None, workspace=None, stream=None):
    """verify_greedy that reads no row after a request's first rejection, in
    windows (see ``window_ends``)."""
    torch = _torch()
    B, K1, V = _shape3(target, "target")
    K = K1 - 1
    dt = _dtype_code(target)
    _validate((target, "target", None, None), (tokens, "tokens", torch.int32, (B, K)),
              (depth, "depth", torch.int32, (B,)), *_out_specs(B, K, out_tokens, num_accepted))
    out_tokens, num_accepted, _, _ = _new_outputs(target.device, B, K, out_tokens, num_accepted)
    ws, nbytes = _ws(target.device, B, K, V, workspace)
    ep, ne, _keep = _ends_arg(window_ends(K, window, ends))
    st = lib.spec_verify_greedy_early_exit(_ptr(target), dt, _ptr(tokens), _ptr(depth),
                                           B, K, V, ep, ne, _ptr(out_tokens), _ptr(num_accepted),
                                           _ptr(ws), nbytes, _stream(stream))
    _raise("spec_verify_greedy_early_exit", st)
    return out_tokens, num_accepted


def verify_sample_early_exit(target, draft, tokens, temperature, u_accept, u_sample, depth=None, *,
                             window=None, ends=None, out_tokens=None, num_accepted=None, p_draft=None,
                             q_draft=None, want_probs: bool = True, workspace=None, stream=None):
    """verify_sample that reads no row after a request's first rejection, in
    windows (see ``window_ends``).  Returns (out_tokens, num_accepted,
    p_draft, q_draft)."""
    B, K1, V = _shape3(target, "target")
    K = K1 - 1
    dt = _dtype_code(target)
    _validate(*_sample_specs(target, draft, tokens, temperature, u_accept, u_sample, depth, B, K, V),
              *_out_specs(B, K, out_tokens, num_accepted, p_draft, q_draft))
    out_tokens, num_accepted, p_draft, q_draft = _new_outputs(target.device, B, K, out_tokens, num_accepted,
                                                              p_draft, q_draft, want_probs)
    ws, nbytes = _ws(target.device, B, K, V, workspace)
    ep, ne, _keep = _ends_arg(window_ends(K, window, ends))
    st = lib.spec_verify_sample_early_exit(_ptr(target), _ptr(draft), dt, _ptr(tokens),
                                           _ptr(depth), _ptr(temperature), _ptr(u_accept), _ptr(u_sample),
                                           B, K, V, ep, ne, _ptr(out_tokens), _ptr(num_accepted),
                                           _ptr(p_draft), _ptr(q_draft), _ptr(ws), nbytes, _stream(stream))
    _raise("spec_verify_sample_early_exit", st)
    return out_tokens, num_accepted, p_draft, q_draft


def draft_confidence(draft, max_depth=None, *, conf=None, workspace=None, stream=None):
    """conf[b,k] = max softmax(draft[b,k]) at T=1 (0 beyond max_depth[b])."""
    torch = _torch()
    B, K, V = _shape3(draft, "draft")
    dt = _dtype_code(draft)
    _validate((draft, "draft", None, None), (max_depth, "max_depth", torch.int32, (B,)),
              (conf, "conf", torch.float32, (B, K)))
    if conf is None:
        conf = torch.empty((B, K), dtype=torch.float32, device=draft.device)
    ws, nbytes = _ws(draft.device, B, K, V, workspace)
    st = lib.spec_draft_confidence(_ptr(draft), dt, _ptr(max_depth), B, K, V, _ptr(conf),
                                   _ptr(ws), nbytes, _stream(stream))
    _raise("spec_draft_confidence", st)
    return conf


def draft_confidence_stats(draft, max_depth=None, *, temperature=None, conf=None, want_conf: bool = True,
                           stats=None, workspace=None, stream=None):
    """Draft confidence plus every read draft row's statistics (sv_row_stat
    records, returned as a float64 tensor [B, K, 2]: see row_stat_fields),
    taken at T = 1, or with `temperature` [B] at each request's own
    temperature (spec_draft_confidence_stats_t).  Returns (conf or None,
    stats)."""
    torch = _torch()
    B, K, V = _shape3(draft, "draft")
    dt = _dtype_code(draft)
    _validate((draft, "draft", None, None), (max_depth, "max_depth", torch.int32, (B,)),
              (temperature, "temperature", torch.float32, (B,)),
              (conf, "conf", torch.float32, (B, K)), (stats, "stats", torch.float64, (B, K, 2)))
    if want_conf and conf is None:
        conf = torch.empty((B, K), dtype=torch.float32, device=draft.device)
    if stats is None:
        stats = torch.empty((B, K, 2), dtype=torch.float64, device=draft.device)
    ws, nbytes = _ws(draft.device, B, K, V, workspace)
    if temperature is None:
        st = lib.spec_draft_confidence_stats(_ptr(draft), dt, _ptr(max_depth), B, K, V,
                                             _ptr(conf), _ptr(stats), _ptr(ws), nbytes, _stream(stream))
        _raise("spec_draft_confidence_stats", st)
    else:
        st = lib.spec_draft_confidence_stats_t(_ptr(draft), dt, _ptr(max_depth), _ptr(temperature), B, K, V,
                                               _ptr(conf), _ptr(stats), _ptr(ws), nbytes, _stream(stream))
        _raise("spec_draft_confidence_stats_t", st)
    return conf, stats


def row_stat_fields(stats):
    """(max float32 [B, K], sum float64 [B, K], temp float32 [B, K]) of
    sv_row_stat records (temp: the temperature they were taken at)."""
    torch = _torch()
    f = stats.view(torch.float32)
    return f[..., 0].contiguous(), stats[..., 1].contiguous(), f[..., 1].contiguous()


def verify_sample_reuse(target, draft, tokens, temperature, u_accept, u_sample, draft_stats, depth=None, *,
                        out_tokens=None, num_accepted=None, p_draft=None, q_draft=None,
                        want_probs: bool = True, workspace=None, stream=None):
    """verify_sample with the draft rows' statistics from draft_confidence_stats
    (used for every sampled request whose statistics were taken at its own
    temperature)."""
    torch = _torch()
    B, K1, V = _shape3(target, "target")
    K = K1 - 1
    dt = _dtype_code(target)
    _validate(*_sample_specs(target, draft, tokens, temperature, u_accept, u_sample, depth, B, K, V),
              (draft_stats, "draft_stats", torch.float64, (B, K, 2)),
              *_out_specs(B, K, out_tokens, num_accepted, p_draft, q_draft))
    out_tokens, num_accepted, p_draft, q_draft = _new_outputs(target.device, B, K, out_tokens, num_accepted,
                                                              p_draft, q_draft, want_probs)
    ws, nbytes = _ws(target.device, B, K, V, workspace)
    st = lib.spec_verify_sample_reuse(_ptr(target), _ptr(draft), dt, _ptr(tokens), _ptr(depth),
                                      _ptr(temperature), _ptr(u_accept), _ptr(u_sample), _ptr(draft_stats),
                                      B, K, V, _ptr(out_tokens), _ptr(num_accepted), _ptr(p_draft),
                                      _ptr(q_draft), _ptr(ws), nbytes, _stream(stream))
    _raise("spec_verify_sample_reuse", st)
    return out_tokens, num_accepted, p_draft, q_draft


# the latency table printed with the pages' cost-aware D-cut sketch (depth: relative cost)
DEFAULT_COST_TABLE = ((1.0, 1.0), (2.0, 1.2), (4.0, 1.5), (8.0, 2.0), (16.0, 3.0))


def _conf_shape(conf):
    torch = _torch()
    if not isinstance(conf, torch.Tensor):
        raise TypeError(f"conf must be a torch tensor, got {type(conf).__name__}")
    if conf.dim() != 2:
        raise ValueError(f"conf must be 2-D [B, K], got shape {tuple(conf.shape)}")
    return int(conf.shape[0]), int(conf.shape[1])


def dcut_allocate_cost(conf, max_verify: float, max_depth=None, table=DEFAULT_COST_TABLE, *,
                       depth_out=None, stream=None):
    """Cost-aware D-cut (per-request best benefit/cost depth, greedy budget fill)."""
    torch = _torch()
    B, K = _conf_shape(conf)
    _validate((conf, "conf", torch.float32, (B, K)), (max_depth, "max_depth", torch.int32, (B,)),
              (depth_out, "depth_out", torch.int32, (B,)))
    if depth_out is None:
        depth_out = torch.empty((B,), dtype=torch.int32, device=conf.device)
    n = len(table)
    td = (ctypes.c_double * n)(*[float(p[0]) for p in table])
    tc = (ctypes.c_double * n)(*[float(p[1]) for p in table])
    st = lib.dcut_allocate_cost(_ptr(conf), _ptr(max_depth), B, K, ctypes.cast(td, ctypes.c_void_p),
                                ctypes.cast(tc, ctypes.c_void_p), n, float(max_verify),
                                _ptr(depth_out), _stream(stream))
    _raise("dcut_allocate_cost", st)
    return depth_out


def accept_stats_update(num_accepted, K: int, depth=None, counters=None, *, stream=None):
    """Adds one call's acceptance statistics into counters (int64 [2K + 4] on
    the device; created zeroed when None) and returns them."""
    torch = _torch()
    if not isinstance(num_accepted, torch.Tensor) or num_accepted.dim() != 1:
        raise ValueError("num_accepted must be a 1-D int32 tensor [B]")
    B = int(num_accepted.shape[0])
    _validate((num_accepted, "num_accepted", torch.int32, (B,)), (depth, "depth", torch.int32, (B,)),
              (counters, "counters", torch.int64, (2 * K + 4,)))
    if counters is None:
        counters = torch.zeros(2 * K + 4, dtype=torch.int64, device=num_accepted.device)
    st = lib.spec_accept_stats_update(_ptr(num_accepted), _ptr(depth), B, K, _ptr(counters), _stream(stream))
    _raise("spec_accept_stats_update", st)
    return counters


def accept_stats_summary(counters, K: int) -> dict:
    """Per-position acceptance, mean accepted length and tau from the counters
    (spec_accept_stats_summary on a host copy of them)."""
    torch = _torch()
    c = counters.detach().cpu() if isinstance(counters, torch.Tensor) else torch.tensor(list(counters))
    c = c.to(torch.int64).contiguous()
    if c.numel() != 2 * K + 4:
        raise ValueError(f"counters must hold 2K + 4 = {2 * K + 4} values, got {c.numel()}")
    alpha = (ctypes.c_double * max(K, 1))()
    mean, tau = ctypes.c_double(0.0), ctypes.c_double(0.0)
    st = lib.spec_accept_stats_summary(ctypes.c_void_p(c.data_ptr()), K, ctypes.cast(alpha, ctypes.c_void_p),
                                       ctypes.byref(mean), ctypes.byref(tau))
    _raise("spec_accept_stats_summary", st)
    v = c.tolist()
    return {"alpha": [alpha[k] for k in range(K)], "reached": v[:K], "accepted": v[K:2 * K],
            "requests": v[2 * K], "bad": v[2 * K + 1], "mean_accepted": mean.value, "tau": tau.value}


def dcut_allocate(conf, budget: int, max_depth=None, *, depth_out=None, stream=None):
    """D-cut depth allocation (global top-k of fp32 prefix confidence)."""
    torch = _torch()
    B, K = _conf_shape(conf)
    _validate((conf, "conf", torch.float32, (B, K)), (max_depth, "max_depth", torch.int32, (B,)),
              (depth_out, "depth_out", torch.int32, (B,)))
    if depth_out is None:
        depth_out = torch.empty((B,), dtype=torch.int32, device=conf.device)
    st = lib.dcut_allocate(_ptr(conf), _ptr(max_depth), B, K, int(budget), _ptr(depth_out), _stream(stream))
    _raise("dcut_allocate", st)
    return depth_out
