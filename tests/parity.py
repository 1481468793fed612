"""GPU-vs-oracle comparison helpers for the parity tests.

Rules (the verification path's stated tolerances):
  * greedy requests: out_tokens and num_accepted bit-exact;
  * sampled requests: p_draft / q_draft within 1e-6 absolute; accept
    decisions and emitted tokens identical except where the oracle's
    |u - min(1, p/q)| < 1e-5 (decision band) or the emitted token is the
    oracle's choice for a uniform within 1e-6 of u on the oracle's own
    normalised CDF (CDF band).  Such excused cases are counted; a request
    whose first difference is excused counts once and is not compared
    further.  Any other difference is a hard mismatch.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

P_TOL = 1e-6
U_BAND = 1e-5
CDF_BAND = 1e-6


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy logits/ints/floats -> contiguous GPU tensor (uint16 = bf16 bits)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class Tally:
    def __init__(self):
        self.rows = 0
        self.requests = 0
        self.excused_accept = 0
        self.excused_cdf = 0
        self.hard = []
        self.max_pq_err = 0.0

    @property
    def excused(self):
        return self.excused_accept + self.excused_cdf

    def assert_ok(self, label=""):
        assert not self.hard, f"{label}: {len(self.hard)} hard mismatches, first: {self.hard[:3]}"
        assert self.max_pq_err <= P_TOL, f"{label}: p/q error {self.max_pq_err}"
        assert self.excused <= 1e-4 * self.rows, \
            f"{label}: excused {self.excused} of {self.rows} rows exceeds 1e-4"


def compare_greedy(w: synth.Workload, out, n, depth=None, tally: Tally | None = None):
    o_out, o_n = oracle.verify_greedy(w.target, w.tokens, depth)
    bad = np.nonzero((o_n != n) | np.any(o_out != out, axis=1))[0]
    if tally is not None:
        d = np.full(w.B, w.K) if depth is None else np.asarray(depth)
        tally.rows += int(np.sum(np.maximum(d, 0) + 1))
        tally.requests += w.B
        for b in bad[:5]:
            tally.hard.append((int(b), "greedy", o_out[b].tolist(), out[b].tolist(), int(o_n[b]), int(n[b])))
    return bad


def compare_sample(w: synth.Workload, out, n, p, q, depth=None, tally: Tally | None = None,
                   ora: dict | None = None) -> Tally:
    tally = tally or Tally()
    if ora is None:
        ora = oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept,
                                   w.u_sample, depth)
    o_out, o_n = ora["out"], ora["n"]
    d_all = np.full(w.B, w.K) if depth is None else np.asarray(depth)
    tally.rows += int(np.sum(np.clip(d_all, 0, None) + 1))
    tally.requests += w.B
    if p is not None:
        tally.max_pq_err = max(tally.max_pq_err, float(np.max(np.abs(p - ora["p_draft"]), initial=0.0)),
                               float(np.max(np.abs(q - ora["q_draft"]), initial=0.0)))
    diff = np.nonzero((o_n != n) | np.any(o_out != out, axis=1))[0]
    for b in diff:
        b = int(b)
        T = float(w.temperature[b])
        if o_n[b] == -1 or n[b] == -1 or T == 0.0:
            tally.hard.append((b, "exact", o_out[b].tolist(), out[b].tolist(), int(o_n[b]), int(n[b])))
            continue
        if n[b] != o_n[b]:
            k = int(min(n[b], o_n[b]))
            if abs(float(w.u_accept[b, k]) - float(ora["ratio"][b, k])) < U_BAND:
                tally.excused_accept += 1
            else:
                tally.hard.append((b, "decision", k, float(w.u_accept[b, k]), float(ora["ratio"][b, k])))
            continue
        nb = int(n[b])
        if not np.array_equal(out[b, :nb], o_out[b, :nb]) or np.any(out[b, nb + 1:] != -1):
            tally.hard.append((b, "prefix", o_out[b].tolist(), out[b].tolist()))
            continue
        d = int(d_all[b])
        if nb < d:
            r, _ = oracle.residual(w.target[b, nb], w.draft[b, nb], T)
        else:
            r, _ = oracle.residual(w.target[b, d], None, T)
        t = int(out[b, nb])
        F = np.cumsum(r) / np.sum(r)
        lo = F[t - 1] if t > 0 else 0.0
        u = float(w.u_sample[b])
        if 0 <= t < r.size and r[t] > 0 and lo - CDF_BAND <= u < F[t] + CDF_BAND:
            tally.excused_cdf += 1
        else:
            tally.hard.append((b, "token", int(o_out[b, nb]), t, u, float(lo), float(F[t]) if 0 <= t < r.size else None))
    return tally


def run_greedy(w: synth.Workload, depth=None, tokens=None):
    import draft_verification_verify_amd as sv
    tok = w.tokens if tokens is None else tokens
    out, n = sv.verify_greedy(dev(w.target), dev(tok), dev(depth))
    torch.cuda.synchronize()
    return host(out), host(n)


def run_sample(w: synth.Workload, depth=None):
    import draft_verification_verify_amd as sv
    out, n, p, q = sv.verify_sample(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                    dev(w.u_accept), dev(w.u_sample), dev(depth))
    torch.cuda.synchronize()
    return host(out), host(n), host(p), host(q)


def run_sample_reuse(w: synth.Workload, depth=None, max_depth=None):
    """Confidence pass with statistics, then verification reusing them."""
    import draft_verification_verify_amd as sv
    _, st = sv.draft_confidence_stats(dev(w.draft), dev(max_depth), want_conf=False)
    out, n, p, q = sv.verify_sample_reuse(dev(w.target), dev(w.draft), dev(w.tokens), dev(w.temperature),
                                          dev(w.u_accept), dev(w.u_sample), st, dev(depth))
    torch.cuda.synchronize()
    return host(out), host(n), host(p), host(q)


# ------------------------------------------------------- packed layout ----

def _poison(dtype):
    """A value no parity case expects to be read: NaN logits (bf16 bits for
    uint16)."""
    return np.uint16(0x7FC0) if dtype == np.uint16 else np.float32(np.nan)


class Packed:
    """Packed (CSR) copy of a padded workload's first depth[b] drafted
    positions per request: offsets o (o_0 = start), target rows (b, 0..d_b)
    at o_b + b + k, draft rows, tokens and accept uniforms (b, k < d_b) at
    o_b + k.  `slack` unused positions follow o_B; unused rows hold NaN and
    unused tokens / uniforms invalid values, so a stray read shows up."""

    def __init__(self, w: synth.Workload, depth, start: int = 0, slack: int = 0, offsets=None):
        d = np.asarray(depth, np.int64)
        B, K, V = w.B, w.K, w.V
        self.depth = d
        if offsets is None:
            offsets = start + np.concatenate([[0], np.cumsum(d)])
        self.offsets = np.asarray(offsets, np.int64).astype(np.int32)
        self.N = int(start + d.sum() + slack)
        N = self.N
        self.target = np.full((N + B, V), _poison(w.target.dtype), w.target.dtype)
        self.draft = np.full((N, V), _poison(w.draft.dtype), w.draft.dtype)
        self.tokens = np.full(N, -7, np.int32)
        self.u_accept = np.full(N, 2.0, np.float32)
        for b in range(B):
            o = int(self.offsets[b])
            db = int(d[b])
            if db < 0 or db > K:
                continue
            self.target[o + b:o + b + db + 1] = w.target[b, :db + 1]
            self.draft[o:o + db] = w.draft[b, :db]
            self.tokens[o:o + db] = w.tokens[b, :db]
            self.u_accept[o:o + db] = w.u_accept[b, :db]

    def unpack(self, w: synth.Workload, out, p=None, q=None):
        """Padded [B, K+1] / [B, K] views of packed outputs (-1 / 0 past each
        request's slots), and the mask of packed output slots no request owns."""
        B, K = w.B, w.K
        out_pad = np.full((B, K + 1), -1, np.int32)
        p_pad = np.zeros((B, K), np.float32)
        q_pad = np.zeros((B, K), np.float32)
        owned = np.zeros(self.N + B, bool)
        for b in range(B):
            o, db = int(self.offsets[b]), int(self.depth[b])
            if db < 0 or db > K:
                continue
            out_pad[b, :db + 1] = out[o + b:o + b + db + 1]
            owned[o + b:o + b + db + 1] = True
            if p is not None:
                p_pad[b, :db] = p[o:o + db]
                q_pad[b, :db] = q[o:o + db]
        return out_pad, p_pad, q_pad, ~owned


def run_greedy_packed(pk: Packed, K_max: int, sentinel: int = -99):
    import draft_verification_verify_amd as sv
    B = pk.offsets.size - 1
    out = torch.full((pk.N + B,), sentinel, dtype=torch.int32, device="cuda")
    num = torch.full((B,), sentinel, dtype=torch.int32, device="cuda")
    sv.verify_greedy_packed(dev(pk.target), dev(pk.tokens), dev(pk.offsets), K_max, out_tokens=out, num_accepted=num)
    torch.cuda.synchronize()
    return host(out), host(num)


def run_sample_packed(pk: Packed, w: synth.Workload, K_max: int, sentinel: int = -99):
    import draft_verification_verify_amd as sv
    B = pk.offsets.size - 1
    out = torch.full((pk.N + B,), sentinel, dtype=torch.int32, device="cuda")
    num = torch.full((B,), sentinel, dtype=torch.int32, device="cuda")
    p = torch.full((pk.N,), -3.0, dtype=torch.float32, device="cuda")
    q = torch.full((pk.N,), -3.0, dtype=torch.float32, device="cuda")
    sv.verify_sample_packed(dev(pk.target), dev(pk.draft), dev(pk.tokens), dev(pk.offsets), dev(w.temperature),
                            dev(pk.u_accept), dev(w.u_sample), K_max, out_tokens=out, num_accepted=num,
                            p_draft=p, q_draft=q)
    torch.cuda.synchronize()
    return host(out), host(num), host(p), host(q)
