"""Benchmark of batched draft verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-secondary]

One step = one spec_verify_sample call (row statistics, accept test,
first-rejection scan, residual/bonus draw, output assembly) over the dense
D-cut workload at full depth: B=64 requests, K=16 drafted tokens, V=128000,
bf16 logits, T=1, every request verified at depth 16 (B*(K+1) = 1088 verified
target rows, 1024 draft rows).  Inputs are seeded synthetic logits already
resident in HBM; input copies are rotated so the 256 MB memory-side cache
cannot serve a step from the previous one.  The K timed steps run back to
back between two events on the launch stream (an event after every call
would add about 2.5 us to each; the spread is taken in a separate pass).

Printed: one JSON line with the verified-rows/s metric, the roofline of the
dominant kernel (the row-statistics pass; its duration from HIP events that
the library records on the launch stream around each kernel of every timed
call), the oracle CPU baseline on a bounded sample, and secondary
measurements (greedy, the K=3 chat shape, the D-cut pipeline, the mixed fp32
batch, early exit).

Profiling helpers (run under rocprofv3; see the summaries under profiles/):
    python bench.py --early-exit-ends 4,16
                                          times only early-exit calls with those
                                          window ends (for kernel traces)
    python bench.py --trace-shape k3      times only the K=3 chat calls (B=4,
                                          sampled, then greedy), for traces
    python bench.py --trace-shape greedy  times only greedy calls on the
                                          headline batch, for traces
    python bench.py --pmc-pass            a few headline steps, then a plain
                                          device copy of 512 MiB (counter
                                          calibration); prints the kernel names
    python bench.py --pmc-summary DIR...  reads rocprofv3 counter CSVs from the
                                          given directories (one FETCH_SIZE run,
                                          one WRITE_SIZE run; no GPU needed) and
                                          prints the scaled per-launch traffic
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "draft_verification_verify_amd", "csrc", "specverify.hip")
ROW_PASS_KERNEL = "row_pass_kernel"
CALIB_BYTES = 512 * 2**20          # fp32 elements read once and written once by the calibration copy
CALIB_KERNEL = "neg_kernel"

# HBM traffic of one row-statistics launch on the headline workload (bytes),
# from two rocprofv3 --pmc runs of `bench.py --pmc-pass` (FETCH_SIZE, then
# WRITE_SIZE), each scaled by what the same counter reads for the calibration
# copy in that run.  It describes the kernel source with this SHA-256 only;
# for any other source it is reported as null.
ROW_PASS_TRAFFIC = {"source_sha256": "c301634da640cb2650df714ccfc883a87e560943efe3e7042756aa82fa0a3537",
                    "fetch_bytes": 525406560, "write_bytes": 897576,
                    # SQ counters of the same source (one --pmc run of eight SQ counters):
                    # VALU instructions and busy cycles per dispatch, summed over the device
                    "sq_insts_valu": 32479039, "sq_busy_cycles": 5713611}


# Untimed steps before the first timed pass (less any --warmup steps).
SETTLE_STEPS = 500


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # measured on MI355X: after 30 warm-up steps the next 100 back-to-back
    # steps still averaged 5-7 us slower than after 500 or 2000 (the GPU had
    # not reached its steady state); 500 steps take about 60 ms
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR")
    ap.add_argument("--early-exit-ends", default="", metavar="E1,E2,...",
                    help="time only early-exit calls with these window ends (for kernel traces)")
    ap.add_argument("--trace-shape", choices=("k3", "greedy"), default="",
                    help="time only the K=3 chat shape (B=4, sampled then greedy) or the greedy headline "
                         "batch, eager calls (for kernel traces)")
    return ap.parse_args()


def source_sha256() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def row_pass_rows(w, mode: str, depth=None) -> int:
    """Logit rows the row-statistics kernel reads: target rows 0..d_b of a
    request verified by the greedy rule; target rows 0..d_b-1 and draft rows
    0..d_b-1 of a sampled request (its target row d_b is read only by a bonus
    draw, in the sampler)."""
    d = np.full(w.B, w.K) if depth is None else np.asarray(depth)
    if mode == "greedy":
        return int(np.sum(d + 1))
    return int(np.sum(np.where(w.temperature > 0, 2 * d, d + 1)))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- pmc summary
def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def pmc_summary(dirs):
    """Per-kernel mean of each counter (KiB per dispatch as rocprofv3 reports
    FETCH_SIZE / WRITE_SIZE), the calibration factor from the plain copy, and
    the scaled bytes per launch of the row-statistics kernel."""
    per = {}
    for d in dirs:
        for r in _counter_rows(d):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            ctr = r.get("Counter_Name") or r.get("Counter-Name")
            val = float(r.get("Counter_Value") or r.get("Counter-Value") or 0.0)
            disp = r.get("Dispatch_Id") or r.get("Dispatch-Id") or r.get("Correlation_Id")
            per.setdefault(ctr, {}).setdefault(name, {}).setdefault(disp, 0.0)
            per[ctr][name][disp] += val       # sum over the rows of one dispatch
    res = {"counters": {}}
    for ctr, kernels in per.items():
        row = [v for n, v in kernels.items() if ROW_PASS_KERNEL in n]
        cal = [v for n, v in kernels.items() if CALIB_KERNEL in n]
        rdc = [v for n, v in kernels.items() if "read_ceiling_kernel" in n]
        if not row or not cal:
            continue
        row_kib = float(np.mean([x for v in row for x in v.values()]))
        cal_kib = float(np.mean([x for v in cal for x in v.values()]))
        factor = CALIB_BYTES / (cal_kib * 1024.0)
        res["counters"][ctr] = {"row_pass_kib_per_dispatch": row_kib, "copy_kib_per_dispatch": cal_kib,
                                "copy_known_bytes": CALIB_BYTES, "scale": factor,
                                "row_pass_bytes_per_launch": row_kib * 1024.0 * factor}
        if rdc:
            # the read-ceiling kernel reads CALIB_BYTES with the row pass's loads
            rd_kib = float(np.mean([x for v in rdc for x in v.values()]))
            res["counters"][ctr]["read_ceiling_kib_per_dispatch"] = rd_kib
            if rd_kib > 0:
                res["counters"][ctr]["read_scale"] = CALIB_BYTES / (rd_kib * 1024.0)
    res["source_sha256"] = source_sha256()
    print(json.dumps(res, indent=1))


# --------------------------------------------------------------------- main
def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: the verification path has no "
                                   "multi-GPU part in this library (requests shard with no exchange)",
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

    # ------------------------------------------------------------------ inputs
    log("generating dense D-cut workload B=64 K=16 V=128000 bf16 (T=1)")
    w = synth.dcut_ragged(args.seed, T=1.0)
    B, K, V = w.B, w.K, w.V
    rows = synth.rows_verified(w)
    algo_bytes = synth.algorithmic_bytes(w, "sample")
    rp_bytes = row_pass_rows(w, "sample") * V * 2
    ncopy = max(2, -(-512 * 2**20 // algo_bytes) + 1)
    log(f"rows/step={rows} algorithmic bytes/step={algo_bytes/1e6:.1f} MB "
        f"(row pass {rp_bytes/1e6:.1f} MB), rotating {ncopy} input copies")
    tgt0, dr0 = dev(w.target), dev(w.draft)
    copies = [(tgt0, dr0)] + [(tgt0.clone(), dr0.clone()) for _ in range(ncopy - 1)]
    tok, T, ua, us = dev(w.tokens), dev(w.temperature), dev(w.u_accept), dev(w.u_sample)
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
    nacc = torch.empty((B,), dtype=torch.int32, device="cuda")
    pd = torch.empty((B, K), dtype=torch.float32, device="cuda")
    qd = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ws = torch.zeros(sv.workspace_size(B, 16, 152064), dtype=torch.uint8, device="cuda")

    def step(i):
        t, d = copies[i % ncopy]
        sv.verify_sample(t, d, tok, T, ua, us, out_tokens=out, num_accepted=nacc, p_draft=pd,
                         q_draft=qd, workspace=ws, stream=stream)

    def timed(fn, steps, warmup, stages=False, per_step=False):
        """Warm up, then time exactly `steps` calls between two events on the
        launch stream (synchronised on both sides), back to back; the mean
        step is returned for every step.  With `per_step`, an event also
        follows every call (about 2.5 us each on MI355X, so only for
        percentiles).  With `stages`, the library also records its per-kernel
        events for every timed call."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        n_ev = steps + 1 if per_step else 2
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        if stages:
            sv.timing_begin(steps)
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(steps):
            fn(i)
            if per_step:
                evs[i + 1].record(stream)
        if not per_step:
            evs[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if per_step:
            per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        else:
            per = [evs[0].elapsed_time(evs[1]) / steps] * steps
        st = sv.timing_end(steps) if stages else None
        return wall, per, st

    if args.pmc_pass:
        # byte counts do not depend on clocks: a few steps suffice
        for i in range(min(max(args.warmup, 1), 30) + max(min(args.steps, 5), 1)):
            step(i)
        src = torch.rand(CALIB_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        # a second calibration read with the row pass's own load instruction
        # (16-byte nontemporal loads): the read-ceiling kernel over the same bytes
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(3):
            sv.read_ceiling(src, sink, stream)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": "done", "row_pass_kernel": ROW_PASS_KERNEL,
                          "calibration": f"torch.neg over {CALIB_BYTES} B of fp32 (reads and writes that many); "
                                         f"read_ceiling_kernel over the same {CALIB_BYTES} B (reads that many)"}))
        return

    if args.early_exit_ends:
        ends = [int(x) for x in args.early_exit_ends.split(",")]

        def estep(i):
            t, d = copies[i % ncopy]
            sv.verify_sample_early_exit(t, d, tok, T, ua, us, ends=ends, out_tokens=out, num_accepted=nacc,
                                        p_draft=pd, q_draft=qd, workspace=ws, stream=stream)
        _, eper, _ = timed(estep, args.steps, args.warmup)
        print(json.dumps({"early_exit_ends": ends, "ms_per_call": float(np.mean(eper)), "steps": args.steps,
                          "mean_accepted": float(nacc.float().mean().item())}))
        return

    if args.trace_shape:
        report = {"trace_shape": args.trace_shape, "steps": args.steps, "warmup": args.warmup}
        if args.trace_shape == "greedy":
            wg = synth.dcut_ragged(args.seed, T=0.0)
            gt = dev(wg.target)
            gcopies = [gt] + [gt.clone() for _ in range(max(2, -(-512 * 2**20 // wg.target.nbytes) + 1) - 1)]
            gtok = dev(wg.tokens)
            _, gper, _ = timed(lambda i: sv.verify_greedy(gcopies[i % len(gcopies)], gtok, out_tokens=out,
                                                          num_accepted=nacc, workspace=ws, stream=stream),
                               args.steps, args.warmup)
            report["greedy_ms_per_call"] = float(np.mean(gper))
        else:
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
                _, cper, _ = timed(cstep, args.steps, args.warmup)
                report[f"k3_{mode}_ms_per_call"] = float(np.mean(cper))
        print(json.dumps(report))
        return

    # The library's per-kernel events (on the launch stream, around each
    # kernel of every timed call) for the roofline's kernel duration; the
    # event markers add a few microseconds per call, so this pass is separate
    # from the headline region.  It runs first, with the plain-read pass, so
    # that the headline region runs on a GPU that has left its idle clocks
    # (after only a few warm-up steps from idle, steps ran 2-5 us slower).
    # Settle: untimed steps before the first timed pass, whatever --warmup
    # says, so that no timed region (the per-kernel pass included) runs on a
    # GPU still leaving its idle clocks.  Measured on MI355X: with 5 warm-up
    # steps the first pass's row pass took 92.6 us against 86.1 us after 500.
    settle = max(SETTLE_STEPS - args.warmup, 0)
    log(f"settling: {settle} untimed steps")
    for i in range(settle):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps with per-kernel events after {args.warmup} warm-up steps")
    _, sper, st = timed(step, args.steps, args.warmup, stages=True)
    st = np.asarray(st, dtype=np.float64)
    stage_ms = st.mean(axis=0)
    rp_ms = float(stage_ms[0])
    achieved = rp_bytes / (rp_ms * 1e-3) / 1e9
    # practical ceiling: a plain read of as many bytes as the row pass reads,
    # alternating two buffers so the 256 MB MALL serves none of it
    log("timing the plain read of the row pass's bytes")
    rbufs = [torch.ones(rp_bytes // 2, dtype=torch.int16, device="cuda") for _ in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, cper, _ = timed(lambda i: sv.read_ceiling(rbufs[i % 2], sink, stream), args.steps, args.warmup)
    ceil_ms = float(np.mean(cper))
    ceil_gbs = rp_bytes / (ceil_ms * 1e-3) / 1e9
    del rbufs
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps (headline)")
    wall, per, _ = timed(step, args.steps, args.warmup)
    # the same steps with an event after each, for the spread only
    _, per_ev, _ = timed(step, args.steps, 2, per_step=True)
    ms = float(np.mean(per))
    value = rows / (ms * 1e-3)
    n_mean = float(nacc.float().mean().item())
    sha = source_sha256()
    traffic = None
    valu_busy = None
    if ROW_PASS_TRAFFIC["source_sha256"] == sha and ROW_PASS_TRAFFIC["fetch_bytes"] is not None:
        traffic = float(ROW_PASS_TRAFFIC["fetch_bytes"] + ROW_PASS_TRAFFIC["write_bytes"])
        # VALU-busy fraction: 4 cycles per wave64 instruction on each of the
        # 1024 SIMDs, against the kernel's cycles (busy cycles summed over the
        # 32 shader engines)
        valu_busy = ROW_PASS_TRAFFIC["sq_insts_valu"] * 4.0 / (1024 * ROW_PASS_TRAFFIC["sq_busy_cycles"] / 32)
    result = {
        "metric": "verified logit rows/sec (B×(K+1) rows of V) + % of HBM peak, K=3 and K=16",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "settle_note": "untimed steps run before the first timed pass (per-kernel events, then the plain "
                       "read, then the headline region with its own --warmup steps)",
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense D-cut verification at full depth: B=64 K=16 V=128000 bf16 logits, "
                               "rejection sampling at T=1, draft noise sigma_b~U(0.3,2.0)",
                   "global_batch": B, "K": K, "V": V, "rows_per_step": rows, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": 100.0 * algo_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": algo_bytes,
        "ms_p10_p50_p90": [float(np.percentile(per_ev, q)) for q in (10, 50, 90)],
        "ms_p10_p50_p90_note": "a second pass of the same steps with an event after each call "
                               "(the events add about 2.5 us per step; ms_per_step has none)",
        "stage_ms": {"row_pass": rp_ms, "finish": float(stage_ms[1]), "draw": float(stage_ms[2]),
                     "step_with_events": float(np.mean(sper))},
        "wall_s_timed": wall,
        "mean_accepted": n_mean,
        "tau_incl_bonus": n_mean + 1.0,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ROW_PASS_KERNEL + "<bf16> (row statistics)",
                     "algorithmic_bytes_per_launch": rp_bytes,
                     "avg_launch_ms": rp_ms, "valu_busy": valu_busy},
        "kernel_source_sha256": sha,
        "read_ceiling": {"GB_s": ceil_gbs, "ms": ceil_ms, "bytes": rp_bytes,
                         "row_pass_frac_of_ceiling": achieved / ceil_gbs,
                         "note": "spec_verify_read_ceiling: one plain read of the row pass's bytes, same load "
                                 "width and cache policy, two alternating buffers"},
    }

    # -------------------------------------------------------------- secondary
    if not args.no_secondary:
        sec = {}
        steps2, warm2 = max(args.steps // 2, 10), max(args.warmup // 2, 3)
        # greedy at full depth, same shape (T=0 drafts are the draft argmax)
        wg = synth.dcut_ragged(args.seed, T=0.0)
        gt = dev(wg.target)
        gcopies = [gt] + [gt.clone() for _ in range(max(2, -(-512 * 2**20 // wg.target.nbytes) + 1) - 1)]
        gtok = dev(wg.tokens)

        def gstep(i):
            sv.verify_greedy(gcopies[i % len(gcopies)], gtok, out_tokens=out, num_accepted=nacc, workspace=ws,
                             stream=stream)
        # the step without event markers, then again with the library's
        # per-kernel events for the row pass's time
        _, gper, _ = timed(gstep, steps2, warm2)
        _, _, gst = timed(gstep, steps2, 2, stages=True)
        gms = float(np.mean(gper))
        gbytes = synth.algorithmic_bytes(wg, "greedy")
        grp = float(np.mean([s[0] for s in gst]))
        sec["greedy_dense_B64_K16"] = {"rows_per_s": rows / (gms * 1e-3), "ms": gms,
                                       "GB_s": gbytes / (gms * 1e-3) / 1e9,
                                       "pct_hbm_peak": 100 * gbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "row_pass_ms": grp,
                                       "row_pass_GB_s": gbytes / (grp * 1e-3) / 1e9}
        # the same greedy batch verified with early exit (default window ends)
        gn_one = nacc.cpu().numpy().copy()
        gends = sv.window_ends(K)

        def gestep(i):
            sv.verify_greedy_early_exit(gcopies[i % len(gcopies)], gtok, ends=gends, out_tokens=out,
                                        num_accepted=nacc, workspace=ws, stream=stream)
        _, geper, _ = timed(gestep, steps2, warm2)
        gems = float(np.mean(geper))
        sec["early_exit_greedy_ends_" + "_".join(map(str, gends)) + "_B64_K16"] = {
            "rows_per_s": rows / (gems * 1e-3), "ms": gems, "vs_one_pass_ms": gms / gems,
            "mean_accepted": float(nacc.float().mean().item()),
            "same_num_accepted_as_one_pass": bool(np.array_equal(nacc.cpu().numpy(), gn_one))}
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
            _, cper, _ = timed(cstep, steps2, warm2)
            cms = float(np.mean(cper))
            _, _, cst = timed(cstep, steps2, 2, stages=True)
            cstage = np.asarray(cst, dtype=np.float64).mean(axis=0)
            # the same calls replayed from a HIP graph (20 calls per graph):
            # GPU time per call without the host's enqueue work in between
            NG = 20

            def cgraph_body(mode=mode):
                for _ in range(NG):
                    if mode == "sample":
                        sv.verify_sample(ct, cd, ctok, cT, cua, cus, out_tokens=cout, num_accepted=cn,
                                         want_probs=False, workspace=ws)
                    else:
                        sv.verify_greedy(ct, ctok, out_tokens=cout, num_accepted=cn, workspace=ws)
            cgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cgraph):
                cgraph_body()
            torch.cuda.synchronize()
            _, gper_c, _ = timed(lambda i: cgraph.replay(), max(steps2 // 4, 5), 3)
            gms_c = float(np.mean(gper_c)) / NG
            del cgraph
            cb = synth.algorithmic_bytes(wc, mode)
            crow = synth.rows_verified(wc)
            sec[f"mtp_chat_B4_K3_{mode}"] = {
                "rows_per_s": crow / (cms * 1e-3), "ms": cms,
                "GB_s": cb / (cms * 1e-3) / 1e9, "pct_hbm_peak": 100 * cb / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "graph_replay_ms_per_call": gms_c, "graph_replay_rows_per_s": crow / (gms_c * 1e-3),
                "stage_ms_with_events": {"row_pass": float(cstage[0]), "finish": float(cstage[1]),
                                         "draw": float(cstage[2])},
                "note": "ms: eager calls back to back through the binding; graph_replay: 20 calls per HIP "
                        "graph, replayed; stage_ms: the library's per-kernel events (each adds ~1 us)"}
        # block drafting for code/math (B=16, K=16), sampled and greedy; its
        # 135 MB fits the 256 MB memory-side cache, so five copies rotate
        for mode in ("sample", "greedy"):
            wb = synth.block_code(args.seed, T=1.0 if mode == "sample" else 0.0)
            bcopies = [(dev(wb.target), dev(wb.draft)) for _ in range(5)]
            btok, bT, bua, bus = dev(wb.tokens), dev(wb.temperature), dev(wb.u_accept), dev(wb.u_sample)
            bout = torch.empty((wb.B, wb.K + 1), dtype=torch.int32, device="cuda")
            bn = torch.empty((wb.B,), dtype=torch.int32, device="cuda")

            def bstep(i, mode=mode):
                bt, bd = bcopies[i % 5]
                if mode == "sample":
                    sv.verify_sample(bt, bd, btok, bT, bua, bus, out_tokens=bout, num_accepted=bn,
                                     want_probs=False, workspace=ws, stream=stream)
                else:
                    sv.verify_greedy(bt, btok, out_tokens=bout, num_accepted=bn, workspace=ws, stream=stream)
            _, bper, _ = timed(bstep, steps2, warm2)
            bms = float(np.mean(bper))
            bbytes = synth.algorithmic_bytes(wb, mode)
            brow = synth.rows_verified(wb)
            sec[f"block_code_B16_K16_{mode}"] = {
                "rows_per_s": brow / (bms * 1e-3), "ms": bms, "GB_s": bbytes / (bms * 1e-3) / 1e9,
                "pct_hbm_peak": 100 * bbytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "mean_accepted": float(bn.float().mean().item()),
                "note": "B=16 K=16 V=128000 bf16, planted +8 targets, calibrated draft-noise ramp; five "
                        "input copies rotated"}
            del bcopies
        # D-cut pipeline: confidence -> dcut_allocate(384) -> ragged sampled verify
        conf = torch.empty((B, K), dtype=torch.float32, device="cuda")
        depth = torch.empty((B,), dtype=torch.int32, device="cuda")

        def pstep(i):
            t, d = copies[i % ncopy]
            sv.draft_confidence(d, conf=conf, workspace=ws, stream=stream)
            sv.dcut_allocate(conf, w.budget, depth_out=depth, stream=stream)
            sv.verify_sample(t, d, tok, T, ua, us, depth, out_tokens=out, num_accepted=nacc, p_draft=pd,
                             q_draft=qd, workspace=ws, stream=stream)
        _, pper, _ = timed(pstep, steps2, warm2)
        pms = float(np.mean(pper))
        dep = depth.cpu().numpy()
        prow = int(np.sum(dep + 1))
        sec["dcut_pipeline_B64_K16_budget384"] = {
            "verified_rows_per_s": prow / (pms * 1e-3), "ms": pms, "rows_per_step": prow,
            "bytes_per_step": int((B * K + prow + int(dep.sum())) * V * 2),
            "note": "confidence pass reads all 1024 draft rows; ragged verify reads sum(d_b+1) target "
                    "and sum(d_b) draft rows"}
        # the allocation alone, on the pipeline's last confidences
        _, aper, _ = timed(lambda i: sv.dcut_allocate(conf, w.budget, depth_out=depth, stream=stream), steps2, warm2)
        sec["dcut_allocate_B64_K16_budget384"] = {
            "ms": float(np.mean(aper)), "keys": B * K,
            "note": "global top-k of fp32 prefix confidence (one workgroup, LDS radix select)"}
        # the ragged verify alone at the D-cut depths: reads sum(d_b + 1)
        # target and sum(d_b) draft rows of the padded buffers
        rsum = int(dep.sum())
        ralgo = (prow + rsum) * V * 2

        def vstep(i):
            t, d = copies[i % ncopy]
            sv.verify_sample(t, d, tok, T, ua, us, depth, out_tokens=out, num_accepted=nacc, p_draft=pd,
                             q_draft=qd, workspace=ws, stream=stream)
        _, vper, _ = timed(vstep, steps2, warm2)
        _, _, vst = timed(vstep, steps2, 2, stages=True)
        vms = float(np.mean(vper))
        vstage = np.asarray(vst, dtype=np.float64).mean(axis=0)
        vrp_bytes = 2 * rsum * V * 2
        sec["dcut_ragged_verify_B64_K16_budget384"] = {
            "verified_rows_per_s": prow / (vms * 1e-3), "ms": vms, "rows_per_step": prow,
            "algorithmic_bytes_per_step": ralgo, "GB_s": ralgo / (vms * 1e-3) / 1e9,
            "pct_hbm_peak": 100 * ralgo / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "stage_ms_with_events": {"row_pass": float(vstage[0]), "finish": float(vstage[1]),
                                     "draw": float(vstage[2])},
            "row_pass_GB_s": vrp_bytes / (float(vstage[0]) * 1e-3) / 1e9,
            "note": "spec_verify_sample alone at the D-cut depths (budget 384): sum(d_b + 1) target and "
                    "sum(d_b) draft rows; padded [B,K+1,V] buffers, rotated"}
        # the same verify on the packed (CSR) layout: the buffers hold only
        # the sum(d_b + 1) target and sum(d_b) draft rows (gathered here,
        # outside the timed region; three copies rotated, 640 MB)
        tgt_idx = torch.tensor([b * (K + 1) + k for b in range(B) for k in range(int(dep[b]) + 1)],
                               dtype=torch.int64, device="cuda")
        drf_idx = torch.tensor([b * K + k for b in range(B) for k in range(int(dep[b]))],
                               dtype=torch.int64, device="cuda")
        offs = torch.tensor(np.concatenate([[0], np.cumsum(dep)]).astype(np.int32), device="cuda")
        pcopies = [(copies[i % ncopy][0].view(B * (K + 1), V)[tgt_idx].contiguous(),
                    copies[i % ncopy][1].view(B * K, V)[drf_idx].contiguous()) for i in range(3)]
        ptok = tok.view(-1)[drf_idx].contiguous()
        pua = ua.view(-1)[drf_idx].contiguous()
        pout = torch.empty(rsum + B, dtype=torch.int32, device="cuda")
        ppd = torch.empty(rsum, dtype=torch.float32, device="cuda")
        pqd = torch.empty(rsum, dtype=torch.float32, device="cuda")

        def kstep(i):
            pt, pdr = pcopies[i % 3]
            sv.verify_sample_packed(pt, pdr, ptok, offs, T, pua, us, K, out_tokens=pout, num_accepted=nacc,
                                    p_draft=ppd, q_draft=pqd, workspace=ws, stream=stream)
        _, kper, _ = timed(kstep, steps2, warm2)
        _, _, kst = timed(kstep, steps2, 2, stages=True)
        kms = float(np.mean(kper))
        kstage = np.asarray(kst, dtype=np.float64).mean(axis=0)
        sec["dcut_packed_verify_B64_K16_budget384"] = {
            "verified_rows_per_s": prow / (kms * 1e-3), "ms": kms, "rows_per_step": prow,
            "algorithmic_bytes_per_step": ralgo, "GB_s": ralgo / (kms * 1e-3) / 1e9,
            "pct_hbm_peak": 100 * ralgo / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "buffer_bytes": int(pcopies[0][0].nbytes + pcopies[0][1].nbytes),
            "stage_ms_with_events": {"row_pass": float(kstage[0]), "finish": float(kstage[1]),
                                     "draw": float(kstage[2])},
            "row_pass_GB_s": vrp_bytes / (float(kstage[0]) * 1e-3) / 1e9,
            "note": "spec_verify_sample_packed at the D-cut depths (budget 384): CSR offsets, buffers of "
                    "sum(d_b + 1) target and sum(d_b) draft rows only; three copies rotated"}
        del pcopies
        # the same pipeline with the confidence pass's row statistics reused:
        # the verify streams target rows only (plus the drawn draft row)
        dstats = torch.empty((B, K, 2), dtype=torch.float64, device="cuda")

        def rstep(i):
            t, d = copies[i % ncopy]
            sv.draft_confidence_stats(d, conf=conf, stats=dstats, workspace=ws, stream=stream)
            sv.dcut_allocate(conf, w.budget, depth_out=depth, stream=stream)
            sv.verify_sample_reuse(t, d, tok, T, ua, us, dstats, depth, out_tokens=out, num_accepted=nacc,
                                   p_draft=pd, q_draft=qd, workspace=ws, stream=stream)
        _, rper, _ = timed(rstep, steps2, warm2)
        rms = float(np.mean(rper))
        rdep = depth.cpu().numpy()
        rrow = int(np.sum(rdep + 1))
        sec["dcut_pipeline_reuse_B64_K16_budget384"] = {
            "verified_rows_per_s": rrow / (rms * 1e-3), "ms": rms, "rows_per_step": rrow,
            "bytes_per_step": int((B * K + int(rdep.sum())) * V * 2),
            "note": "confidence pass (with row statistics) reads all 1024 draft rows; the verify reuses "
                    "them and streams sum(d_b) target rows"}
        # cost-aware D-cut on the same confidences (the pages' latency table), alone
        cdep = torch.empty((B,), dtype=torch.int32, device="cuda")

        def cstep2(i):
            sv.dcut_allocate_cost(conf, 96.0, depth_out=cdep, stream=stream)
        _, cper2, _ = timed(cstep2, steps2, warm2)
        sec["dcut_allocate_cost_B64_K16"] = {
            "ms": float(np.mean(cper2)), "admitted": int((cdep > 0).sum().item()),
            "verify_slots": int(cdep.sum().item()),
            "note": "max_verify 96 in the table's cost units (1.0 at depth 1 ... 3.0 at depth 16); one workgroup; on these high-entropy drafts every request's best benefit/cost depth is 1"}
        # early-exit verification of the same dense batch: windows ending at
        # the given positions, no row read after a request's first rejection;
        # the committed tokens are those of the one-pass step
        step(0)
        n_one = nacc.cpu().numpy().copy()
        # the window ends planned from this batch's measured per-position
        # acceptance (device counters -> spec_early_exit_plan, window cost
        # 2.5 positions)
        cnt = sv.accept_stats_update(nacc, K)
        alpha = sv.accept_stats_summary(cnt, K)["alpha"]
        planned = sv.early_exit_plan(alpha, 2.5)
        schedules = [[4, 16], [2, 6, 16], [1, 16], [8, 16], [4, 8, 12, 16]]
        if planned not in schedules:
            schedules.append(planned)
        sec["early_exit_planned_ends"] = {"ends": planned, "window_cost": 2.5,
                                          "alpha": [round(a, 4) for a in alpha]}
        for ends in schedules:
            def estep(i, ends=ends):
                t, d = copies[i % ncopy]
                sv.verify_sample_early_exit(t, d, tok, T, ua, us, ends=ends, out_tokens=out, num_accepted=nacc,
                                            p_draft=pd, q_draft=qd, workspace=ws, stream=stream)
            _, eper, _ = timed(estep, steps2, warm2)
            ems = float(np.mean(eper))
            en = nacc.cpu().numpy()
            # positions whose target and draft rows the row passes stream:
            # up to the end of the window in which the request stops
            pos_read = [K if n >= K else min(K, next(e for e in ends if e > n)) for n in en.tolist()]
            sec["early_exit_ends_" + "_".join(map(str, ends)) + "_B64_K16"] = {
                "rows_per_s": rows / (ems * 1e-3), "ms": ems, "vs_one_pass_ms": ms / ems,
                "row_pass_rows_per_step": 2 * int(sum(pos_read)), "one_pass_row_pass_rows": 2 * B * K,
                "windows": len(ends), "same_num_accepted_as_one_pass": bool(np.array_equal(en, n_one)),
                "note": "rows_per_s counts the B*(K+1) rows the step decides, as the headline does; "
                        "the row passes stream the positions up to the end of each request's stopping "
                        "window"}
        del copies
        # mixed fp32 batch: per-request K_b and T_b, dcut_allocate(512), one sampled launch
        wm = synth.mixed(args.seed)
        mt0, md0 = dev(wm.target), dev(wm.draft)
        # two copies of 1.28 GB each: the 256 MB memory-side cache serves none of a step
        mcopies = [(mt0, md0), (mt0.clone(), md0.clone())]
        mtok, mT, mua, mus = dev(wm.tokens), dev(wm.temperature), dev(wm.u_accept), dev(wm.u_sample)
        mK = dev(wm.max_depth)
        mconf = torch.empty((wm.B, wm.K), dtype=torch.float32, device="cuda")
        mdep = torch.empty((wm.B,), dtype=torch.int32, device="cuda")
        mout = torch.empty((wm.B, wm.K + 1), dtype=torch.int32, device="cuda")
        mn = torch.empty((wm.B,), dtype=torch.int32, device="cuda")

        def mstep(i):
            mt, md = mcopies[i % 2]
            sv.draft_confidence(md, mK, conf=mconf, workspace=ws, stream=stream)
            sv.dcut_allocate(mconf, wm.budget, mK, depth_out=mdep, stream=stream)
            sv.verify_sample(mt, md, mtok, mT, mua, mus, mdep, out_tokens=mout, num_accepted=mn,
                             want_probs=False, workspace=ws, stream=stream)
        _, mper, _ = timed(mstep, steps2, warm2)
        mms = float(np.mean(mper))
        mdv = mdep.cpu().numpy()
        mrow = int(np.sum(mdv + 1))
        sec["mixed_fp32_B64_V152064_budget512"] = {
            "verified_rows_per_s": mrow / (mms * 1e-3), "ms": mms, "rows_per_step": mrow,
            "note": "confidence over all max_depth draft rows + dcut_allocate + one mixed-K/T sampled launch; "
                    "two input copies rotated"}
        # the same pipeline with the confidence pass's draft-row statistics
        # reused, taken at T = 1 (only requests at T = 1 skip their draft rows
        # in the verify) and at each request's own temperature (every sampled
        # request skips them)
        mst = torch.empty((wm.B, wm.K, 2), dtype=torch.float64, device="cuda")
        Tm = wm.temperature
        row_b = wm.V * 4
        d_t1 = int(np.sum(mdv[Tm == 1.0]))
        d_tx = int(np.sum(mdv[(Tm > 0) & (Tm != 1.0)]))
        for tag, temps in (("T1", None), ("any_T", mT)):
            def mrstep(i, temps=temps):
                mt, md = mcopies[i % 2]
                sv.draft_confidence_stats(md, mK, temperature=temps, conf=mconf, stats=mst, workspace=ws,
                                          stream=stream)
                sv.dcut_allocate(mconf, wm.budget, mK, depth_out=mdep, stream=stream)
                sv.verify_sample_reuse(mt, md, mtok, mT, mua, mus, mst, mdep, out_tokens=mout, num_accepted=mn,
                                       want_probs=False, workspace=ws, stream=stream)
            _, mrper, _ = timed(mrstep, steps2, warm2)
            mrms = float(np.mean(mrper))
            reused = d_t1 if temps is None else d_t1 + d_tx
            sec[f"mixed_fp32_reuse_{tag}_B64_V152064_budget512"] = {
                "verified_rows_per_s": mrow / (mrms * 1e-3), "ms": mrms, "vs_no_reuse_ms": mms / mrms,
                "draft_rows_reused": reused, "draft_rows_streamed": d_t1 + d_tx - reused,
                "bytes_saved_per_step": reused * row_b,
                "note": ("spec_draft_confidence_stats (statistics at T = 1: requests at T = 0.7 still stream "
                         "their d_b draft rows)" if temps is None else
                         "spec_draft_confidence_stats_t (statistics at each request's temperature, two sums "
                         "per row at T != 1)") + " + dcut_allocate + spec_verify_sample_reuse; T = 0 requests "
                         "read no draft rows"}
        del mcopies, mt0, md0
        result["secondary"] = sec

    # ----------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        log("timing the CPU oracle on the same workload (all 64 requests, repeated to >= 10 s)")
        reps, t_tot = 0, 0.0
        while t_tot < 10.0 and reps < 8:
            t0 = time.perf_counter()
            oracle.verify_sample(w.target, w.draft, w.tokens, w.temperature, w.u_accept, w.u_sample)
            t_tot += time.perf_counter() - t0
            reps += 1
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
        except OSError:
            pass
        result["cpu_baseline"] = {"value": reps * rows / t_tot, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the full headline batch (64 requests, {rows} verified rows) "
                                            f"run {reps} times in {t_tot:.1f} s; single-threaded C, fp64",
                                  "cpu": f"1 core of {os.cpu_count()} visible, {cpu_model}"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
