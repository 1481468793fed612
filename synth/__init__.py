"""Seeded synthetic verification workloads.

The pages measure speculative decoding on public benchmarks and on
production traffic ([Stack] = aimodeling.com, "Tencent Hunyuan Turns
Speculative Decoding Into a Full Open-Source Stack", section "Key numbers";
[Hamidun] = news.hamidun.com, "Tencent открыл AngelSpec ...", per-position
acceptance paragraph).  None of that data is available here.  These generators
stand in for it with random logits of the same shapes:
  * MTP depth 3 for chat ([Stack], section "Five angles worth a closer look",
    item 5: the Hy3 MTP drafter is trained with TTT over 3 steps);
  * block drafts for code and math (the DFly block drafter; block size 8 in
    the deep-dive's drafter listing, 16 here);
  * a 128000-token vocabulary (the vocabulary size of the deep-dive's MTP and
    DFly listings; 152064 for the mixed batch);
  * concurrency 4 to 64 ([Stack], section "Key numbers").

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the verification arithmetic: it draws logits, draft tokens and
uniforms, nothing else.  Draft tokens at T > 0 are drawn by the Gumbel-max
trick (argmax of logits/T plus Gumbel noise), which samples softmax(y/T)
without evaluating a softmax; at T = 0 they are the draft's argmax (a greedy
drafter).

Per-depth draft-noise levels that hit the acceptance targets are read from
``noise_calibration.json``, written by ``synth/calibrate.py`` (which uses the
oracle only).

Seeds: numpy ``default_rng(SeedSequence([20261203, workload_id, stream,
seed]))`` with streams 0 target, 1 draft noise, 2 draft-token noise,
3 u_accept, 4 u_sample, 5 per-request parameters.  bf16 values are fp32
draws rounded to nearest-even and stored as the upper 16 bits (uint16).
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20261203
S_TARGET, S_NOISE, S_TOKENS, S_UACC, S_USAMP, S_PARAMS = range(6)

_CAL_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noise_calibration.json")

# Workload ids (first element of the seed sequence after the base).
W_TINY, W_MTP_CHAT, W_BLOCK_CODE, W_DCUT, W_MIXED, W_FUZZ = 1, 2, 3, 4, 5, 9


def rng(workload: int, stream: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, workload, stream, seed]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest, ties to even) stored as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Stored logits (uint16 bf16 bits or float32) widened exactly to float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


@dataclass
class Workload:
    name: str
    dtype: str                 # "bf16" (uint16 storage) or "f32"
    target: np.ndarray         # [B, K+1, V]
    draft: np.ndarray          # [B, K, V]
    tokens: np.ndarray         # [B, K] int32
    temperature: np.ndarray    # [B] float32
    u_accept: np.ndarray       # [B, K] float32 in [0, 1)
    u_sample: np.ndarray       # [B] float32 in [0, 1)
    max_depth: np.ndarray      # [B] int32, K_b (drafted tokens available per request)
    budget: int | None = None  # D-cut budget (verified drafted positions), if any
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.target.shape[0]

    @property
    def K(self) -> int:
        return self.target.shape[1] - 1

    @property
    def V(self) -> int:
        return self.target.shape[2]

    def nbytes(self) -> int:
        return self.target.nbytes + self.draft.nbytes


def load_calibration() -> dict:
    with open(_CAL_PATH) as f:
        return json.load(f)


def _draft_tokens(draft_f64_row: np.ndarray, T: float, g: np.random.Generator) -> int:
    """One drafted token: argmax (T = 0) or a Gumbel-max sample of softmax(y/T)."""
    if T == 0.0:
        return int(np.argmax(draft_f64_row))
    u = g.random(draft_f64_row.shape[0])
    with np.errstate(divide="ignore"):
        gumbel = -np.log(-np.log(u))
    return int(np.argmax(draft_f64_row / T + gumbel))


def _uniforms(wid: int, seed: int, B: int, K: int):
    ua = rng(wid, S_UACC, seed).random((B, K), dtype=np.float32)
    us = rng(wid, S_USAMP, seed).random(B, dtype=np.float32)
    return ua, us


def _normal_target(g, V, scale):
    return (g.standard_normal(V, dtype=np.float32) * np.float32(scale))


def _planted_target(g, V, boost):
    z = g.standard_normal(V, dtype=np.float32)
    j = int(g.integers(0, V))
    z[j] += np.float32(boost)
    return z


def build(name: str, dtype: str, B: int, K: int, V: int, *, wid: int, seed: int,
          target_fn, sigma_fn, temperature: np.ndarray, max_depth: np.ndarray | None = None,
          budget: int | None = None, pad_nan: bool = False, meta: dict | None = None) -> Workload:
    """Generic generator.

    target_fn(b, g) -> fp32 [V] logits for one target row of request b.
    sigma_fn(b, k) -> draft-noise std for draft row k of request b; the draft
    row is the stored target row plus N(0, sigma^2) noise.
    Rows outside a request's K_b window are filled with NaN when pad_nan is
    set, so that reading them is detectable."""
    if max_depth is None:
        max_depth = np.full(B, K, np.int32)
    gt, gn, gx = rng(wid, S_TARGET, seed), rng(wid, S_NOISE, seed), rng(wid, S_TOKENS, seed)
    sdt = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((B, K + 1, V), sdt)
    draft = np.empty((B, K, V), sdt)
    tokens = np.zeros((B, K), np.int32)
    for b in range(B):
        Kb = int(max_depth[b])
        T = float(temperature[b])
        for k in range(K + 1):
            if k <= Kb:
                target[b, k] = _store(target_fn(b, gt), dtype)
            else:
                target[b, k] = _store(np.full(V, np.nan, np.float32), dtype) if pad_nan else target[b, k - 1]
        for k in range(K):
            if k < Kb:
                t32 = bf16_bits_to_f32(target[b, k]) if dtype == "bf16" else target[b, k]
                noise = gn.standard_normal(V, dtype=np.float32) * np.float32(sigma_fn(b, k))
                draft[b, k] = _store(t32 + noise, dtype)
                tokens[b, k] = _draft_tokens(as_f64(draft[b, k]), T, gx)
            else:
                draft[b, k] = _store(np.full(V, np.nan, np.float32), dtype) if pad_nan else draft[b, max(k - 1, 0)]
                tokens[b, k] = 0
    ua, us = _uniforms(wid, seed, B, K)
    return Workload(name, dtype, target, draft, tokens, np.asarray(temperature, np.float32),
                    ua, us, np.asarray(max_depth, np.int32), budget, meta or {})


# ----------------------------------------------------------------------------
# The five workloads.  Each takes a seed and the temperature the run uses; T
# decides how draft tokens are drawn (sampled for T > 0, argmax for T = 0).
# Sizes may be overridden for parity tests at reduced scale.
# ----------------------------------------------------------------------------

def tiny(seed: int = 0, T: float = 1.0, B: int = 1, K: int = 3, V: int = 1000) -> Workload:
    """B=1, K=3, V=1000 fp32; target N(0, 2^2); draft = target + N(0, 0.5^2);
    draft tokens sampled from softmax(draft) at T=1 and reused for T=0 runs."""
    w = build("tiny", "f32", B, K, V, wid=W_TINY, seed=seed,
              target_fn=lambda b, g: _normal_target(g, V, 2.0),
              sigma_fn=lambda b, k: 0.5,
              temperature=np.ones(B, np.float32))
    w.temperature[:] = T
    return w


def mtp_chat(seed: int = 0, T: float = 1.0, B: int = 4, K: int = 3, V: int = 128000,
             literal: bool = False) -> Workload:
    """B=4, K=3, V=128000 bf16; target N(0, 3^2); draft noise per depth tuned so
    T=1 acceptance is about (0.81, 0.66, 0.52) (the chat profile of the
    deep-dive's workload analyser, read per position).  literal=True uses the
    config's stated sigma = 1.0 at every depth instead."""
    if literal:
        sig = [1.0] * K
    else:
        cal = load_calibration()["mtp_chat"]["sigma"]
        sig = [cal[min(k, len(cal) - 1)] for k in range(K)]
    return build("mtp_chat" + ("_literal" if literal else ""), "bf16", B, K, V, wid=W_MTP_CHAT,
                 seed=seed, target_fn=lambda b, g: _normal_target(g, V, 3.0),
                 sigma_fn=lambda b, k: sig[k], temperature=np.full(B, T, np.float32))


def block_code(seed: int = 0, T: float = 1.0, B: int = 16, K: int = 16, V: int = 128000,
               boost: float = 8.0) -> Workload:
    """B=16, K=16, V=128000 bf16; N(0,1) background with one planted token per
    row boosted by +8 (boost=14 gives the peaked variant); draft noise ramped
    per depth so T=1 acceptance falls about linearly from 0.90 to 0.60."""
    cal = load_calibration()["block_code"]["sigma"]
    sig = [cal[min(k, len(cal) - 1)] for k in range(K)]
    return build("block_code" + ("" if boost == 8.0 else f"_boost{boost:g}"), "bf16", B, K, V,
                 wid=W_BLOCK_CODE, seed=seed, target_fn=lambda b, g: _planted_target(g, V, boost),
                 sigma_fn=lambda b, k: sig[k], temperature=np.full(B, T, np.float32))


def dcut_ragged(seed: int = 0, T: float = 1.0, B: int = 64, K: int = 16, V: int = 128000,
                budget: int = 384) -> Workload:
    """B=64, K=16, V=128000 bf16; target N(0, 3^2); per-request constant draft
    noise sigma_b ~ U(0.3, 2.0); D-cut budget 384 verified drafted tokens."""
    sig_b = rng(W_DCUT, S_PARAMS, seed).uniform(0.3, 2.0, B)
    w = build("dcut_ragged", "bf16", B, K, V, wid=W_DCUT, seed=seed,
              target_fn=lambda b, g: _normal_target(g, V, 3.0),
              sigma_fn=lambda b, k: float(sig_b[b]), temperature=np.full(B, T, np.float32),
              budget=budget, meta={"sigma_b": sig_b})
    return w


def mixed(seed: int = 0, B: int = 64, K: int = 16, V: int = 152064, budget: int = 512,
          k_mtp: int = 3) -> Workload:
    """B=64, V=152064 fp32, padded to K=16: half MTP-style requests (K_b=3,
    target N(0, 3^2), draft noise 1.0) and half block-style (K_b=16, planted
    +8 targets, the block workload's draft-noise ramp), in seeded order, with
    per-request T drawn from {0, 0.7, 1.0} and a D-cut budget of 512.  Rows
    beyond a request's K_b are NaN so that any read of them shows up."""
    gp = rng(W_MIXED, S_PARAMS, seed)
    kinds = np.array([0] * (B // 2) + [1] * (B - B // 2))
    gp.shuffle(kinds)
    temps = gp.choice(np.array([0.0, 0.7, 1.0], np.float32), B).astype(np.float32)
    max_depth = np.where(kinds == 0, min(k_mtp, K), K).astype(np.int32)
    cal = load_calibration()["block_code"]["sigma"]

    def target_fn(b, g):
        return _normal_target(g, V, 3.0) if kinds[b] == 0 else _planted_target(g, V, 8.0)

    def sigma_fn(b, k):
        return 1.0 if kinds[b] == 0 else cal[min(k, len(cal) - 1)]

    return build("mixed", "f32", B, K, V, wid=W_MIXED, seed=seed, target_fn=target_fn,
                 sigma_fn=sigma_fn, temperature=temps, max_depth=max_depth, budget=budget,
                 pad_nan=True, meta={"kinds": kinds})


def random_case(seed: int, B: int, K: int, V: int, dtype: str = "bf16", temps=(1.0,),
                scale: float = 3.0, sigma: float = 0.7, wid: int = W_FUZZ, shift: float = 0.0,
                temperature=None) -> Workload:
    """Generic case for parity sweeps: N(0, scale^2) targets plus a constant
    `shift` (rounded to the storage type with each logit), draft noise sigma,
    per-request T drawn from `temps` (or given per request as `temperature`)."""
    gp = rng(wid, S_PARAMS, seed)
    if temperature is None:
        T = gp.choice(np.asarray(temps, np.float32), B).astype(np.float32)
    else:
        T = np.asarray(temperature, np.float32).reshape(B)
    sh = np.float32(shift)
    return build(f"random_{dtype}_{B}x{K}x{V}", dtype, B, K, V, wid=wid, seed=seed,
                 target_fn=lambda b, g: _normal_target(g, V, scale) + sh,
                 sigma_fn=lambda b, k: sigma, temperature=T)


def planted_alpha(seed: int, B: int, alphas, V: int = 16, scale: float = 1.0) -> Workload:
    """Planted per-position acceptance (fp32).  Token w = V-1 has target logit
    -inf; the target over the other tokens is p = softmax(N(0, scale^2)); the
    draft puts mass alpha_j on p and 1 - alpha_j on w, i.e. draft logits
    log(alpha_j) + log p_v and log(1 - alpha_j) at w.  Under the rejection
    rule each drafted token is accepted with probability exactly alpha_j, so
    E[accepted] = sum_k prod_{j<=k} alpha_j.  The log-probabilities are built
    here in float64 and stored as float32 logits; this is input construction,
    the test states the closed form it expects."""
    K = len(alphas)
    g = rng(W_FUZZ + 1, S_TARGET, seed)
    gx = rng(W_FUZZ + 1, S_TOKENS, seed)
    target = np.empty((B, K + 1, V), np.float32)
    draft = np.empty((B, K, V), np.float32)
    tokens = np.empty((B, K), np.int32)
    w = V - 1
    for b in range(B):
        for k in range(K + 1):
            z = g.standard_normal(V) * scale
            z[w] = -np.inf
            target[b, k] = z.astype(np.float32)
        for k in range(K):
            z = target[b, k].astype(np.float64)
            m = np.max(z[:w])
            logp = z[:w] - m - np.log(np.sum(np.exp(z[:w] - m)))
            y = np.empty(V)
            y[:w] = np.log(alphas[k]) + logp
            y[w] = np.log1p(-alphas[k])
            draft[b, k] = y.astype(np.float32)
            tokens[b, k] = _draft_tokens(draft[b, k].astype(np.float64), 1.0, gx)
    ua, us = _uniforms(W_FUZZ + 1, seed, B, K)
    return Workload("planted_alpha", "f32", target, draft, tokens, np.ones(B, np.float32),
                    ua, us, np.full(B, K, np.int32), None, {"alphas": list(alphas)})


def rows_verified(w: Workload, depth: np.ndarray | None = None) -> int:
    """Verified logit rows = sum_b (d_b + 1) (the metric's unit)."""
    d = np.full(w.B, w.K) if depth is None else np.asarray(depth)
    return int(np.sum(d + 1))


def algorithmic_bytes(w: Workload, mode: str, depth: np.ndarray | None = None) -> int:
    """Bytes the method must read: each logit of every verified window once.
    greedy: target rows 0..d_b; sampled: target rows 0..d_b plus draft rows
    0..d_b-1 of requests with T_b > 0 (T_b = 0 requests read no draft rows)."""
    esz = 2 if w.dtype == "bf16" else 4
    d = np.full(w.B, w.K) if depth is None else np.asarray(depth)
    rows = np.sum(d + 1)
    if mode == "sample":
        rows += np.sum(np.where(w.temperature > 0, d, 0))
    return int(rows) * w.V * esz
