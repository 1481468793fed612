"""Find per-depth draft-noise levels that hit the workloads' acceptance targets.

Writes ``synth/noise_calibration.json``.  It uses only the CPU oracle (its
softmax) to evaluate the T=1 acceptance probability of a draft row,
sum_v min(p_v, q_v) -- the probability that the rejection test accepts a
token drawn from q -- averaged over seeded rows built with the generator's
own recipe, and bisects the noise level per position.

Targets:
  mtp_chat   : (0.81, 0.66, 0.52), the chat profile's first three rates in the
               deep-dive's workload analyser (happyrock.cloud, "Tencent
               AngelSpec Speculative Decoding Framework Deep Dive ...",
               WorkloadAnalyzer listing), read per position.
  block_code : linear from 0.90 to 0.60 over 16 positions (the block
               workload's stated per-position acceptance range).

Run:  python -m synth.calibrate
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import synth  # noqa: E402

V = 128000
ROWS = 8


def _rows(kind: str, seed: int):
    g = synth.rng(100 + (0 if kind == "normal" else 1), synth.S_TARGET, seed)
    out = []
    for _ in range(ROWS):
        z = synth._normal_target(g, V, 3.0) if kind == "normal" else synth._planted_target(g, V, 8.0)
        out.append(synth.to_bf16_bits(z))
    return out


def acceptance(kind: str, sigma: float, seed: int = 0) -> float:
    gn = synth.rng(110, synth.S_NOISE, seed)
    acc = []
    for zb in _rows(kind, seed):
        z32 = synth.bf16_bits_to_f32(zb)
        yb = synth.to_bf16_bits(z32 + gn.standard_normal(V, dtype=np.float32) * np.float32(sigma))
        p, _, _ = oracle.softmax(zb, 1.0)
        q, _, _ = oracle.softmax(yb, 1.0)
        acc.append(float(np.minimum(p, q).sum()))
    return float(np.mean(acc))


def solve(kind: str, alpha: float, lo: float = 0.01, hi: float = 6.0, iters: int = 16) -> float:
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if acceptance(kind, mid) > alpha:
            lo = mid
        else:
            hi = mid
    return round(0.5 * (lo + hi), 4)


def main() -> None:
    oracle.build(force=False)
    chat_alpha = [0.81, 0.66, 0.52]
    block_alpha = [round(0.90 - 0.30 * k / 15, 4) for k in range(16)]
    out = {
        "note": "T=1 acceptance sum_v min(p,q) per position; sigma is the std of the Gaussian "
                "noise added to the stored target logits; evaluated by the oracle on 8 seeded "
                "V=128000 bf16 rows per point; written by synth/calibrate.py",
        "mtp_chat": {"alpha": chat_alpha, "sigma": [solve("normal", a) for a in chat_alpha]},
        "block_code": {"alpha": block_alpha, "sigma": [solve("planted", a) for a in block_alpha]},
    }
    for key in ("mtp_chat", "block_code"):
        out[key]["achieved"] = [round(acceptance("normal" if key == "mtp_chat" else "planted", s), 4)
                                for s in out[key]["sigma"]]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noise_calibration.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
