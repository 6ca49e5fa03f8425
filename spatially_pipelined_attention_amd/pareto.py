"""Per-user against per-GPU decode throughput over batch size and schedule.

The SubGPU Pipelining paper (section 5, its throughput frontier figure)
compares schedules by the frontier of tokens/s per user against tokens/s per
GPU. One iteration gives every sequence one token, so a schedule that takes
t ms per iteration at batch B serves 1000 / t tokens/s to each user and
1000 B / t tokens/s per GPU. For every batch this measures the temporal
schedules T_m and the spatial grid (cut x CU split x m, via
spa_pipeline_tune), then keeps the points no other point beats on both axes:

    python -m spatially_pipelined_attention_amd.pareto --workload gptoss_36l_fp8 \\
        --batches 16,64,256,1024 --out pareto.json
"""
from __future__ import annotations

import argparse
import json
import sys
import time
from typing import List


def frontier(points: List[dict]) -> List[dict]:
    """Points not dominated on (per_user, per_gpu), both higher-better,
    sorted by per-user throughput."""
    keep = []
    for p in points:
        dominated = any(q is not p and q["per_user"] >= p["per_user"] and q["per_gpu"] >= p["per_gpu"]
                        and (q["per_user"] > p["per_user"] or q["per_gpu"] > p["per_gpu"]) for q in points)
        if not dominated:
            keep.append(p)
    return sorted(keep, key=lambda p: p["per_user"])


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="gptoss_36l_fp8")
    ap.add_argument("--batches", default="16,64,256,1024")
    ap.add_argument("--micros", default="1,2,4,8")
    ap.add_argument("--cuts", default="0,1,2")
    ap.add_argument("--cu-step", type=int, default=32)
    ap.add_argument("--cu-min", type=int, default=32)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--per-kind", type=int, default=0, choices=(0, 1),
                    help="1: search stage A's CUs for full and sliding layers separately")
    ap.add_argument("--out", required=True)
    ap.add_argument("--virtual-comm", default="", metavar="LATENCY_US,GBPS",
                    help="add the rank's communication endpoints to every layer")
    a = ap.parse_args(argv)

    import torch
    from . import binding as B, synth
    from .workload import DeviceWorkload, parse_comm, set_comm

    base = synth.WORKLOADS[a.workload]
    ctx = B.spa_init(0)
    cuts = [int(x) for x in a.cuts.split(",")][:3]
    comm = parse_comm(a.virtual_comm)
    result = {"workload": a.workload, "n_cus": B.spa_device_cus(ctx), "batches": {},
              "virtual_comm": {"latency_us": comm[0], "gbps": comm[1]} if comm else None}
    points = []
    for bsz in [int(x) for x in a.batches.split(",")]:
        wl = base.with_(batch=bsz)
        micros = [int(x) for x in a.micros.split(",") if bsz % int(x) == 0 and bsz // int(x) * wl.top_k <= 4096][:4]
        t0 = time.time()
        dw = DeviceWorkload(wl)
        if comm:
            set_comm(dw.m, *comm)
        torch.cuda.synchronize()
        setup = time.time() - t0
        ws = max((dw.workspace(n_micro=mm) for mm in micros), key=lambda t: t.numel())
        sp = B.spa_tune_space(len(cuts), (B.C.c_int32 * 3)(*(cuts + [0] * (3 - len(cuts)))),
                              len(micros), (B.C.c_int32 * 4)(*(micros + [0] * (4 - len(micros)))),
                              a.cu_step, a.cu_min, a.warmup, a.reps, 1, a.per_kind)
        t0 = time.time()
        best, pts = B.spa_pipeline_tune(ctx, dw.m, dw.layers_c, dw.batch, ws, sp, torch.cuda.current_stream())
        tune_s = time.time() - t0
        rows = []
        for p in pts:
            r = {"batch": bsz, "schedule": "temporal" if p.cu_a == 0 else "spatial", "cut": p.cut,
                 "n_micro": p.n_micro, "cu_a": p.cu_a, "cu_a_sliding": p.cu_a_sliding, "ms": round(p.ms, 4),
                 "per_user": round(1000.0 / p.ms, 2), "per_gpu": round(1000.0 * bsz / p.ms, 1)}
            rows.append(r)
        temporal = {r["n_micro"]: r for r in rows if r["schedule"] == "temporal"}
        spatial = [r for r in rows if r["schedule"] == "spatial"]
        best_sp = min(spatial, key=lambda r: r["ms"]) if spatial else None
        best_t = min(temporal.values(), key=lambda r: r["ms"])
        result["batches"][str(bsz)] = {
            "temporal_ms": {str(k): v["ms"] for k, v in sorted(temporal.items())},
            "best_temporal": best_t, "best_spatial": best_sp, "points": len(rows),
            "setup_s": round(setup, 1), "tune_s": round(tune_s, 1)}
        print(f"[batch {bsz}] T: " + ", ".join(f"m={k} {v['ms']:.3f}" for k, v in sorted(temporal.items()))
              + (f"; best spatial cut={best_sp['cut']} m={best_sp['n_micro']} cu_a={best_sp['cu_a']}"
                 f"/{best_sp['cu_a_sliding']} "
                 f"{best_sp['ms']:.3f} ms" if best_sp else "") + f" ({len(rows)} points, {tune_s:.0f} s)",
              flush=True)
        points += rows
        del dw, ws
        torch.cuda.empty_cache()
    result["frontier_all"] = frontier(points)
    result["frontier_temporal"] = frontier([p for p in points if p["schedule"] == "temporal"])
    with open(a.out, "w") as f:
        json.dump(result, f, indent=1)
    print("| per-user tok/s | per-GPU tok/s | batch | schedule | cut | m | CUs A | ms |")
    print("|---:|---:|---:|---|---:|---:|---:|---:|")
    for p in result["frontier_all"]:
        cut = p["cut"] if p["schedule"] == "spatial" else "-"
        print(f"| {p['per_user']} | {p['per_gpu']} | {p['batch']} | {p['schedule']} | {cut} | "
              f"{p['n_micro']} | {p['cu_a'] or '-'} | {p['ms']} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
