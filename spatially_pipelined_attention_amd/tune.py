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
    d = json.load(open(a.out)) if os.path.exists(a.out) else {}
    d[key] = entry
    with open(a.out, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
