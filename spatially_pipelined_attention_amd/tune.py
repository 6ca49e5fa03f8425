"""Offline tuning of the spatial pipeline for one workload (section 4 of the
SubGPU Pipelining paper: search offline, select the stored configuration at
run time). Runs spa_pipeline_tune on the GPU with the workload's own inputs
and writes the best spatial point, the temporal times and the selection (the
faster of the two kinds) to a JSON file, merged with what is there:

    python -m spatially_pipelined_attention_amd.tune --workload gptoss_36l_b64 --out tuned.json

With --virtual-comm LATENCY_US,GBPS every layer also runs the rank's
communication endpoints (spa_model_desc.comm_*), and the entry is stored
under "<workload>+comm".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="gptoss_36l_b64")
    ap.add_argument("--out", required=True)
    ap.add_argument("--micros", default="1,2,4")
    ap.add_argument("--cuts", default="0,1,2")
    ap.add_argument("--cu-step", type=int, default=32)
    ap.add_argument("--cu-min", type=int, default=32)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--per-kind", type=int, default=1, help="separate CU splits for full and sliding layers")
    ap.add_argument("--virtual-comm", default="", metavar="LATENCY_US,GBPS")
    ap.add_argument("--points-md", default="", metavar="PATH",
                    help="also write every measured point as a markdown table (with --command as its provenance)")
    ap.add_argument("--command", default="")
    ap.add_argument("--no-store", action="store_true", help="do not merge the result into --out")
    a = ap.parse_args(argv)

    import torch
    from . import binding as B, synth
    from .workload import DeviceWorkload, parse_comm, set_comm

    wl = synth.WORKLOADS[a.workload]
    micros = [int(x) for x in a.micros.split(",") if wl.batch % int(x) == 0][:4]
    cuts = [int(x) for x in a.cuts.split(",")][:3]
    dw = DeviceWorkload(wl)
    comm = parse_comm(a.virtual_comm)
    if comm:
        set_comm(dw.m, *comm)
    key = a.workload + ("+comm" if comm else "")
    ctx = B.spa_init(0)
    ws = max((dw.workspace(n_micro=mm) for mm in micros), key=lambda t: t.numel())
    sp = B.spa_tune_space(len(cuts), (B.C.c_int32 * 3)(*(cuts + [0] * (3 - len(cuts)))),
                          len(micros), (B.C.c_int32 * 4)(*(micros + [0] * (4 - len(micros)))),
                          a.cu_step, a.cu_min, a.warmup, a.reps, 1, a.per_kind)
    t0 = time.time()
    best, pts = B.spa_pipeline_tune(ctx, dw.m, dw.layers_c, dw.batch, ws, sp, torch.cuda.current_stream())
    dt = time.time() - t0
    temporal = {p.n_micro: p.ms for p in pts if p.cu_a == 0}
    # run-time selection among the stored configurations: the best spatial
    # point, or a temporal schedule when one is faster
    t_m, t_ms = min(temporal.items(), key=lambda kv: kv[1])
    selected = {"schedule": "spatial", "n_micro": best.n_micro} if best.ms <= t_ms else \
        {"schedule": "temporal", "n_micro": t_m}
    entry = {"cut": best.cut, "n_micro": best.n_micro, "cu_a": best.cu_a, "cu_a_sliding": best.cu_a_sliding,
             "ms": round(best.ms, 4),
             "temporal_ms": {str(k): round(v, 4) for k, v in sorted(temporal.items())},
             "selected": selected,
             "points": len(pts), "tune_seconds": round(dt, 1), "n_cus": B.spa_device_cus(ctx)}
    if comm:
        entry["virtual_comm"] = {"latency_us": comm[0], "gbps": comm[1]}
    for p in pts:
        print(f"cut={p.cut:2d} m={p.n_micro} cu_a={p.cu_a:3d}/{p.cu_a_sliding:3d}: {p.ms:.3f} ms", flush=True)
    print(json.dumps({key: entry}), flush=True)
    if a.points_md:
        write_points_md(a.points_md, key, wl, pts, best, temporal, a.command or " ".join(sys.argv),
                        B.spa_device_cus(ctx))
    if not a.no_store:
        d = json.load(open(a.out)) if os.path.exists(a.out) else {}
        d[key] = entry
        with open(a.out, "w") as f:
            json.dump(d, f, indent=1, sort_keys=True)
    return 0


def write_points_md(path, key, wl, pts, best, temporal, command, n_cus):
    """Every measured point of a tuning run: temporal schedules and the
    spatial grid (cut x stage-A CUs x microbatches), median iteration ms."""
    t1 = temporal.get(1)
    cut_name = {0: "attn | MoE", 1: "attn+router | experts", 2: "Macro (full attention | rest)"}
    with open(path, "w") as f:
        f.write(f"# Schedule sweep: {key}\n\ncommand: `{command}`\n\n")
        f.write(f"{wl.n_layers} layer(s) ({', '.join(sorted(set(wl.layer_kinds)))}), batch {wl.batch}, "
                f"KV U[{wl.kv_len_lo},{wl.kv_len_hi}], {wl.n_resident} resident experts of {wl.n_experts} "
                f"(top-{wl.top_k}), {wl.expert_dtype} experts. Median of the timed iterations per point.\n\n")
        f.write(f"- temporal_T1_ms: {t1:.4f}\n" if t1 else "")
        f.write(f"- best_spatial_ms: {best.ms:.4f}\n")
        f.write(f"- best_spatial: cut {best.cut}, m {best.n_micro}, stage A {best.cu_a} CUs"
                + (f" (sliding layers {best.cu_a_sliding})" if best.cu_a_sliding != best.cu_a else "") + "\n")
        if t1:
            f.write(f"- best_spatial_vs_T1: {100 * (best.ms / t1 - 1):+.1f}%\n")
        f.write("\n| schedule | cut | m | stage A CUs | stage B CUs | ms | vs T1 |\n|---|---|---:|---:|---:|---:|---:|\n")
        for p in pts:
            kind = "temporal" if p.cu_a == 0 else "spatial"
            cut = "-" if p.cu_a == 0 else cut_name.get(p.cut, str(p.cut))
            a_cus = "-" if p.cu_a == 0 else (str(p.cu_a) if p.cu_a_sliding == p.cu_a else f"{p.cu_a}/{p.cu_a_sliding}")
            b_cus = "-" if p.cu_a == 0 else str(n_cus - p.cu_a)
            rel = f"{100 * (p.ms / t1 - 1):+.1f}%" if t1 else ""
            f.write(f"| {kind} | {cut} | {p.n_micro} | {a_cus} | {b_cus} | {p.ms:.3f} | {rel} |\n")


if __name__ == "__main__":
    sys.exit(main())
