"""Benchmark of batched draft verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one spec_verify_sample call (row statistics, accept test,
first-rejection scan, residual/bonus draw, output assembly) over the dense
D-cut workload at full depth: B=64 requests, K=16 drafted tokens, V=128000,
bf16 logits, T=1, every request verified at depth 16 (B*(K+1) = 1088 target
rows and 1024 draft rows per step).  Inputs are seeded synthetic logits
already resident in HBM; input copies are rotated so the 256 MB
memory-side cache cannot serve a step from the previous one.

Printed: one JSON line with the verified-rows/s metric, the roofline of the
dominant kernel (HIP events on the launch stream), the oracle CPU baseline on
a bounded sample, and secondary measurements (greedy, K=3 chat shape, and
the D-cut pipeline: confidence + dcut_allocate(384) + ragged verify).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; multi-GPU runs are not part of "
                                   "this build (requests shard with no exchange; see the design notes)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import draft_verification_verify_amd as sv
    import synth

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    torch.cuda.init()
    stream = torch.cuda.current_stream()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------------ inputs
    log("generating dense D-cut workload B=64 K=16 V=128000 bf16 (T=1)")
    w = synth.dcut_ragged(args.seed, T=1.0)
    B, K, V = w.B, w.K, w.V
    rows = synth.rows_verified(w)
    algo_bytes = synth.algorithmic_bytes(w, "sample")
    working = algo_bytes
    ncopy = max(2, -(-512 * 2**20 // working) + 1)
    log(f"rows/step={rows} algorithmic bytes/step={algo_bytes/1e6:.1f} MB, rotating {ncopy} input copies")
    tgt0, dr0 = dev(w.target), dev(w.draft)
    copies = [(tgt0, dr0)] + [(tgt0.clone(), dr0.clone()) for _ in range(ncopy - 1)]
    tok, T, ua, us = dev(w.tokens), dev(w.temperature), dev(w.u_accept), dev(w.u_sample)
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    nacc = torch.empty((B,), dtype=torch.int32, device="cuda")
    pd = torch.empty((B, K), dtype=torch.float32, device="cuda")
    qd = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ws = torch.zeros(sv.workspace_size(B, K, V), dtype=torch.uint8, device="cuda")

    def step(i):
        t, d = copies[i % ncopy]
        sv.verify_sample(t, d, tok, T, ua, us, out_tokens=out, num_accepted=nacc, p_draft=pd,
                         q_draft=qd, workspace=ws, stream=stream)

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(steps):
            fn(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        return wall, per

    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    wall, per = timed(step, args.steps, args.warmup)
    ms = float(np.mean(per))
    value = rows / (ms * 1e-3)
    n_mean = float(host_mean(nacc))
    achieved = algo_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "verified logit rows/sec (B×(K+1) rows of V) + % of HBM peak, K=3 and K=16",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense D-cut verification at full depth: B=64 K=16 V=128000 bf16, "
                               "rejection sampling at T=1, draft noise sigma_b~U(0.3,2.0)",
                   "global_batch": B, "K": K, "V": V, "rows_per_step": rows, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBS,
        "ms_p10_p50_p90": [float(np.percentile(per, q)) for q in (10, 50, 90)],
        "wall_s_timed": wall,
        "mean_accepted": n_mean,
        "tau_incl_bonus": n_mean + 1.0,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "whole spec_verify_sample call (row pass + 2 sampler kernels)",
                     "algorithmic_bytes_per_launch": algo_bytes},
    }

    # -------------------------------------------------------------- secondary
    if not args.no_secondary:
        sec = {}
        # greedy at full depth, same shape (T=0 drafts are the draft argmax)
        wg = synth.dcut_ragged(args.seed, T=0.0)
        gt = dev(wg.target)
        gcopies = [gt] + [gt.clone() for _ in range(max(2, -(-512 * 2**20 // wg.target.nbytes) + 1) - 1)]
        gtok = dev(wg.tokens)

        def gstep(i):
            sv.verify_greedy(gcopies[i % len(gcopies)], gtok, out_tokens=out, num_accepted=nacc, workspace=ws,
                             stream=stream)
        _, gper = timed(gstep, args.steps, args.warmup)
        gms = float(np.mean(gper))
        gbytes = synth.algorithmic_bytes(wg, "greedy")
        sec["greedy_dense_B64_K16"] = {"rows_per_s": rows / (gms * 1e-3), "ms": gms,
                                       "GB_s": gbytes / (gms * 1e-3) / 1e9,
                                       "pct_hbm_peak": 100 * gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del gcopies, gt
        # K=3 chat shape (B=4), sampled and greedy
        for mode in ("sample", "greedy"):
            wc = synth.mtp_chat(args.seed, T=1.0 if mode == "sample" else 0.0)
            ct, cd = dev(wc.target), dev(wc.draft)
            ctok, cT, cua, cus = dev(wc.tokens), dev(wc.temperature), dev(wc.u_accept), dev(wc.u_sample)
            cout = torch.empty((wc.B, wc.K + 1), dtype=torch.int32, device="cuda")
            cn = torch.empty((wc.B,), dtype=torch.int32, device="cuda")

            def cstep(i, mode=mode):
                if mode == "sample":
                    sv.verify_sample(ct, cd, ctok, cT, cua, cus, out_tokens=cout, num_accepted=cn,
                                     want_probs=False, workspace=ws, stream=stream)
                else:
                    sv.verify_greedy(ct, ctok, out_tokens=cout, num_accepted=cn, workspace=ws, stream=stream)
            _, cper = timed(cstep, args.steps, args.warmup)
            cms = float(np.mean(cper))
            cb = synth.algorithmic_bytes(wc, mode)
            crow = synth.rows_verified(wc)
            sec[f"mtp_chat_B4_K3_{mode}"] = {"rows_per_s": crow / (cms * 1e-3), "ms": cms,
                                             "GB_s": cb / (cms * 1e-3) / 1e9,
                                             "pct_hbm_peak": 100 * cb / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # D-cut pipeline: confidence -> dcut_allocate(384) -> ragged sampled verify
        conf = torch.empty((B, K), dtype=torch.float32, device="cuda")
        depth = torch.empty((B,), dtype=torch.int32, device="cuda")

        def pstep(i):
            t, d = copies[i % ncopy]
            sv.draft_confidence(d, conf=conf, workspace=ws, stream=stream)
            sv.dcut_allocate(conf, w.budget, depth_out=depth, stream=stream)
            sv.verify_sample(t, d, tok, T, ua, us, depth, out_tokens=out, num_accepted=nacc, p_draft=pd,
                             q_draft=qd, workspace=ws, stream=stream)
        _, pper = timed(pstep, args.steps, args.warmup)
        pms = float(np.mean(pper))
        dep = depth.cpu().numpy()
        prow = int(np.sum(dep + 1))
        sec["dcut_pipeline_B64_K16_budget384"] = {
            "verified_rows_per_s": prow / (pms * 1e-3), "ms": pms, "rows_per_step": prow,
            "bytes_per_step": int((B * K + prow + int(dep.sum())) * V * 2),
            "note": "confidence pass reads all 1024 draft rows; ragged verify reads sum(d_b+1) target "
                    "and sum(d_b) draft rows"}
        result["secondary"] = sec

    # ----------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        nreq = 4
        log(f"timing the CPU oracle on {nreq} of the {B} requests")
        t0 = time.perf_counter()
        oracle.verify_sample(w.target[:nreq], w.draft[:nreq], w.tokens[:nreq], w.temperature[:nreq],
                             w.u_accept[:nreq], w.u_sample[:nreq])
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": nreq * (K + 1) / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{nreq} of the 64 requests of the same workload "
                                            f"({nreq * (K + 1)} verified rows, {dt:.1f} s), single-threaded C, fp64"}
    print(json.dumps(result), flush=True)


def host_mean(t):
    return float(t.float().mean().item())


if __name__ == "__main__":
    main()
