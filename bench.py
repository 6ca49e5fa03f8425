"""Decode-iteration benchmark of the spatially pipelined MoE decode layer.

One step = one 36-layer decode iteration (every layer: Norm+QKV+KV append,
attention, output projection, router, experts, combine) over the resident
batch of the GPT-OSS-shaped one-GPU workload, inputs already in HBM.

Schedules timed (same kernels, same work):
  temporal  T1 : every kernel on all CUs, one microbatch;
  temporal  Tm : the pipeline's microbatches, one after another, all CUs;
  spatial      : two-stage pipeline on disjoint CU pools (cut, CU split, m),
                 as tuned offline (spatially_pipelined_attention_amd/tuned.json).
With --schedule auto (the default) the three are timed and the fastest is
the one run for the reported `value`, as an engine would select among its
stored configurations; all three times are reported beside it. --quick runs
only the stored selection. --schedule spatial / temporal force one.

--virtual-comm LATENCY_US,GBPS adds one rank's communication endpoints to
every layer (attention all-reduce, MoE dispatch, MoE combine; each a kernel
lasting latency + payload / bandwidth, as in the single-GPU emulation of a
32-GPU deployment in section 5.3.1 of the SubGPU Pipelining paper) and uses
the configuration tuned with them ("<workload>+comm").

Prints one JSON line (see the keys below). --gpus N > 1 exits: the pipeline
partitions the CUs of one device.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "36-layer decode iteration µs + achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
TUNED = os.path.join(ROOT, "spatially_pipelined_attention_amd", "tuned.json")


def traffic_from_profile(name, tokens_per_launch):
    """HBM bytes per launch of the full-layer attention kernel from the committed
    counter summary, or None when the kernel's sources or its launch shape (the
    tokens of one microbatch) changed since. The counters are taken on the
    temporal schedule with the same microbatches: its attention launches are
    the spatial pipeline's, on one stream."""
    from spatially_pipelined_attention_amd import profiling
    path = os.path.join(ROOT, "profiles", f"k_attn_full_{name}_traffic.md")
    keys = profiling.read_keys(path)
    if "traffic_bytes_per_launch" not in keys:
        return None, path
    srcs = [os.path.join(ROOT, p.strip()) for p in keys.get("kernel_sources", "").split(",") if p.strip()]
    if not srcs or keys.get("kernel_source_digest") != profiling.source_digest(srcs):
        return None, path
    if keys.get("tokens_per_launch") != str(tokens_per_launch):
        return None, path
    return float(keys["traffic_bytes_per_launch"]), path


DEAL_MAX_TOKENS = 1024   # full-layer launches of up to this many tokens split their KV blocks evenly (kDealMaxTok)


def attn_kernel_name(tokens_per_launch, full=True, n_kv_heads=8, n_cus=256):
    """The attention kernel a launch of this many tokens runs (full or sliding layers)."""
    if not full:   # one wave per window from half a window per CU of the device, the QKV finish folded in
        return "spa::k_attn_wave<1>" if 2 * tokens_per_launch * n_kv_heads >= n_cus else "spa::k_attn<1, 0>"
    if tokens_per_launch <= 256:   # one token per prologue thread
        return "spa::k_attn_dealt<1, 1>"
    return "spa::k_attn_dealt<1, 4>" if tokens_per_launch <= DEAL_MAX_TOKENS else "spa::k_attn<1, 1>"


def load_resample(name):
    p = os.path.join(ROOT, "tests", "golden", f"resample_{name}.json")
    if not os.path.exists(p):
        return {}
    d = json.load(open(p))
    return {int(k): int(v) for k, v in d["resample"].items()}


def tuned_config(name, comm=False):
    if os.path.exists(TUNED):
        d = json.load(open(TUNED))
        for key in ([name + "+comm"] if comm else []) + [name]:
            if key in d:
                return d[key]
    return {"cut": 0, "n_micro": 2, "cu_a": 128}


def dense_weight_bytes(wl):
    """One layer's dense projection and router weights."""
    wb = 2 if wl.w_dtype == "bf16" else 4
    return (wl.qkv_rows * wl.hidden + wl.hidden * wl.n_q_heads * wl.head_dim) * wb + wl.n_experts * wl.hidden * 4


def algorithmic_bytes(dw, n_micro=1):
    """Bytes one iteration of a schedule with n_micro microbatches must move:
    every layer's dense and router weights and the experts that receive rows
    (all resident experts here), once per microbatch; the attended KV window
    of every sequence; and the new K/V rows written."""
    wl = dw.wl
    wb = 2 if wl.w_dtype == "bf16" else 4
    eb = {"bf16": 2, "f32": 4, "e4m3": 1}[wl.expert_dtype]
    H, I, QD = wl.hidden, wl.inter, wl.n_q_heads * wl.head_dim
    dense = dense_weight_bytes(wl)
    experts = wl.n_resident * 3 * H * I * eb
    if wl.expert_dtype == "e4m3":
        experts += wl.n_resident * (2 * I + H) * 4
    per_layer_w = dense + experts
    kv = sum(dw.algorithmic_kv_bytes(l) for l in range(wl.n_layers))
    return wl.n_layers * per_layer_w * n_micro + kv, wl.n_layers * per_layer_w * n_micro, kv


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_iteration_s(name, n_layers=None):
    """Seconds of oracle layer compute for the whole batch over the first
    n_layers layers (all by default); input generation is not timed."""
    from oracle import layer as ol
    from spatially_pipelined_attention_amd import synth
    from tests import harness as hz
    wl = synth.WORKLOADS[name]
    toks = list(range(wl.batch))
    L = synth.kv_lengths(wl)[toks]
    x = synth.x_rows(wl, toks, load_resample(name))
    dt = 0.0
    for l in range(n_layers or wl.n_layers):
        dense = synth.dense_weights(wl, l)
        experts = {e: synth.expert_weights(wl, l, e) for e in range(wl.n_resident)}
        hist = {}
        for bi, b in enumerate(toks):
            lo, hi = ol.attention_window(wl.layer_kinds[l], int(L[bi]), wl.window)
            hist[bi] = (lo, synth.kv_history(wl, l, b, lo, hi - 1))

        def history(bi, lo, hi):
            lo0, (K, V) = hist[bi]
            return K[:, lo - lo0: hi - lo0], V[:, lo - lo0: hi - lo0]
        t0 = time.perf_counter()
        rec = ol.layer_forward(hz.dims(wl), hz.numerics(wl), wl.layer_kinds[l], x, dense, experts.__getitem__, L,
                               history)
        dt += time.perf_counter() - t0
        x = rec.x_next
        del hist
    return dt


def cpu_baseline(name, single_thread_layers=8):
    """The CPU oracle (oracle/: float64 numpy, as written for checking, not
    tuned for speed) on the host cores: the whole iteration for every
    sequence with the BLAS thread pool at its default size, and the first
    `single_thread_layers` layers (half sliding, half full) on one thread,
    scaled to the whole iteration."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS[name]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    dt_all = _oracle_iteration_s(name)
    n1 = min(single_thread_layers, wl.n_layers)
    with threadpool_limits(limits=1):
        dt_one = _oracle_iteration_s(name, n1) * wl.n_layers / n1
    return {"value": dt_all * 1e6, "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole {wl.n_layers}-layer iteration for all {wl.batch} sequences (layer compute timed, "
                      f"input generation excluded), {dt_all:.1f} s with {threads} BLAS threads",
            "single_thread_us": round(dt_one * 1e6, 0),
            "single_thread_sample": f"first {n1} of {wl.n_layers} layers on one thread, scaled x{wl.n_layers / n1:g}",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "impl": "float64 numpy oracle of the tests (not the tuned C++ baseline a production comparison would use)"}


def probe_ceiling():
    """The device's practical HBM read rate from the committed probe summary
    (spatially_pipelined_attention_amd/hbm_probe.py), or None."""
    from spatially_pipelined_attention_amd import profiling
    keys = profiling.read_keys(os.path.join(ROOT, "profiles", "hbm_read_probe.md"))
    return float(keys["ceiling_GBps"]) if "ceiling_GBps" in keys else None


def touched_expert_bytes(dw, n_micro):
    """Bytes of the resident experts that received rows, per microbatch, from
    the picks recorded by the last run (pick t runs expert t % E_res)."""
    wl = dw.wl
    eb = {"bf16": 2, "f32": 4, "e4m3": 1}[wl.expert_dtype]
    per_expert = 3 * wl.hidden * wl.inter * eb + ((2 * wl.inter + wl.hidden) * 4 if wl.expert_dtype == "e4m3" else 0)
    picks = dw.topk.cpu().numpy() % wl.n_resident        # [layers][batch][k]
    bm = wl.batch // n_micro
    n = sum(len(np.unique(picks[l, mu * bm:(mu + 1) * bm])) for l in range(wl.n_layers) for mu in range(n_micro))
    return n * per_expert


TIMER_NOTE = {
    "clock": "device wall clock: first dispatched workgroup's start to the latest workgroup end, recorded by the kernel",
    "events": "HIP events recorded around each launch on its stream",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gptoss_36l_b64")
    ap.add_argument("--batch", type=int, default=None,
                    help="resident sequences (the workload's own by default; other batches skip the CPU baseline "
                         "and the stored router re-draws)")
    ap.add_argument("--schedule", choices=["auto", "spatial", "temporal"], default="auto")
    ap.add_argument("--cut", type=int, default=None)
    ap.add_argument("--micro", type=int, default=None)
    ap.add_argument("--cu-a", type=int, default=None, help="CUs of stage A (multiple of 8)")
    ap.add_argument("--cu-a-sliding", type=int, default=None, help="CUs of stage A in sliding layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the comparison schedules")
    ap.add_argument("--kernel-timer", choices=["clock", "events"], default="clock",
                    help="attention launch duration: the kernel's own span on the device wall clock, or HIP "
                         "events around each launch (these also hold the start marker's dispatch latency)")
    ap.add_argument("--virtual-comm", default="", metavar="LATENCY_US,GBPS",
                    help="add one rank's communication endpoints to every layer (e.g. 3,900)")
    ap.add_argument("--handoff", choices=["values", "events"], default="values",
                    help="stage hand-offs of the spatial pipeline: stream value waits (the default) or events "
                         "(for per-dispatch counter collection, which can hold a value wait's writer back)")
    ap.add_argument("--graph", type=int, choices=[0, 1], default=0,
                    help="temporal schedules replay each iteration from a captured HIP graph (1) or launch "
                         "every kernel directly (0, the faster here: 6.38 against 6.79 ms per 36-layer T1 "
                         "iteration); spatial schedules always launch directly")
    ap.add_argument("--head", type=int, choices=[0, 1], default=0,
                    help="the MoE head (output projection finish .. gather) as separate launches (0, the faster "
                         "here) or as one persistent launch where it applies (1)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES device bytes three times (a known-size kernel for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the pipeline partitions the CUs of a single device; use --gpus 1"}))
        sys.exit(2)

    import torch
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload, Pipeline, parse_comm, set_comm

    name = args.workload
    wl = synth.WORKLOADS[name]
    if args.batch is not None and args.batch != wl.batch:
        wl = wl.with_(batch=args.batch)
        args.no_cpu_baseline = True
    comm = parse_comm(args.virtual_comm)
    cfg = dict(tuned_config(name, comm is not None))
    if args.cut is not None:
        cfg["cut"] = args.cut
    if args.micro is not None:
        cfg["n_micro"] = args.micro
    if args.cu_a is not None:
        cfg["cu_a"] = args.cu_a
        cfg["cu_a_sliding"] = args.cu_a
    if args.cu_a_sliding is not None:
        cfg["cu_a_sliding"] = args.cu_a_sliding
    m = cfg["n_micro"]

    t_setup = time.perf_counter()
    dw = DeviceWorkload(wl, load_resample(name) if wl.batch == synth.WORKLOADS[name].batch else None)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    if comm:
        set_comm(dw.m, *comm)
    ctx = B.spa_init(0)
    n_cus = B.spa_device_cus(ctx)
    ws = dw.workspace(n_micro=m)
    ws1 = dw.workspace(n_micro=1)
    stream = torch.cuda.current_stream()

    def make_pipe(cut, n_micro, cu_a, cu_s=None):
        return Pipeline(ctx, dw.m, {"cut": cut, "n_micro": n_micro, "cu_a": cu_a or 0, "cu_a_sliding": cu_s,
                                    "handoff": 1 if args.handoff == "events" else 0, "graph": args.graph,
                                    "head": args.head})

    results = {}

    def run_schedule(label, cut, n_micro, cu_a, wsx, timed_cls=None, steps=args.steps, warmup=args.warmup, cu_s=None):
        pipe = make_pipe(cut, n_micro, cu_a, cu_s)
        run = lambda: B.spa_pipeline_run(pipe.h, dw.layers_c, dw.batch, wsx, stream)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        if timed_cls is not None:
            B.spa_pipeline_time_kernel(pipe.h, timed_cls, 1 if args.kernel_timer == "clock" else 2)
        torch.cuda.synchronize()
        # a decode step needs the previous step's outputs, so steps are not
        # overlapped: each one is enqueued after the previous one completed
        t0 = time.perf_counter()
        marks = []
        for _ in range(steps):
            run()
            torch.cuda.synchronize()
            marks.append(time.perf_counter())
        ms = (marks[-1] - t0) / steps * 1e3
        step_ms = np.diff(np.array([t0] + marks)) * 1e3
        kt = B.spa_pipeline_timing(pipe.h) if timed_cls is not None else (None, 0)
        pipe.close()
        results[label] = {"ms": ms, "kernel_ms": kt[0], "kernel_n": kt[1],
                          "step_ms": {"mean": round(float(step_ms.mean()), 4), "std": round(float(step_ms.std()), 4),
                                      "min": round(float(step_ms.min()), 4), "max": round(float(step_ms.max()), 4)}}
        return ms, kt

    # comparison schedules first (clean timing), then the reported one with the
    # attention-kernel timer live inside its timed region
    cu_s = cfg.get("cu_a_sliding") or cfg["cu_a"]
    sp_label = (f"spatial cut={cfg['cut']} m={m} cu_a={cfg['cu_a']}/{n_cus}"
                + ("" if cu_s == cfg["cu_a"] else f" (sliding layers {cu_s}/{n_cus})"))
    schedule = args.schedule
    if schedule == "auto":
        if args.quick:
            sel = cfg.get("selected", {"schedule": "spatial"})
            schedule = sel["schedule"]
            if schedule == "temporal":
                m = int(sel.get("n_micro", 1))
        else:
            t1 = run_schedule("temporal_T1", 0, 1, None, ws1)[0]
            tm = run_schedule(f"temporal_T{m}", cfg["cut"], m, None, ws)[0] if m > 1 else t1
            tsp = run_schedule("spatial", cfg["cut"], m, cfg["cu_a"], ws, cu_s=cfg.get("cu_a_sliding"))[0]
            best = min((t1, "temporal", 1), (tm, "temporal", m), (tsp, "spatial", m))
            schedule = best[1]
            m = best[2]
    elif not args.quick:
        run_schedule("temporal_T1", 0, 1, None, ws1)
        if m > 1:
            run_schedule(f"temporal_T{m}", cfg["cut"], m, None, ws)
        if schedule == "temporal":
            run_schedule("spatial", cfg["cut"], m, cfg["cu_a"], ws, cu_s=cfg.get("cu_a_sliding"))
    # the roofline kernel: full-layer attention (sliding-layer attention when the workload has no full layer)
    has_full = "full" in wl.layer_kinds
    attn_cls = B.KC_ATTN_FULL if has_full else B.KC_ATTN_SLIDING
    wsr = ws1 if m == 1 else (ws if m == cfg["n_micro"] else dw.workspace(n_micro=m))
    if schedule == "spatial":
        ms, (k_ms, k_n) = run_schedule("reported", cfg["cut"], m, cfg["cu_a"], wsr, timed_cls=attn_cls,
                                       cu_s=cfg.get("cu_a_sliding"))
        sched = sp_label
    else:   # temporal with the selected (or configured) microbatch count
        ms, (k_ms, k_n) = run_schedule("reported", cfg["cut"], m, None, wsr, timed_cls=attn_cls)
        sched = f"temporal m={m}"
    if args.schedule == "auto":
        sched += " (the fastest of " + ", ".join(k for k in results if k != "reported") + ")" if not args.quick \
            else " (the stored selection)"
    ws = wsr
    errs = B.spa_workspace_errors(ctx, ws)
    if args.copy_calibration > 0:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    total_b, w_b, kv_b = algorithmic_bytes(dw, m)
    min_b = algorithmic_bytes(dw, 1)[0]
    if wl.n_resident > wl.top_k * wl.batch // m or wl.n_resident > 4:
        # many resident experts: only those that received rows are read
        all_e = algorithmic_bytes(dw, 1)[1] - wl.n_layers * dense_weight_bytes(wl)   # every resident expert, once
        total_b += touched_expert_bytes(dw, m) - all_e * m
        min_b += touched_expert_bytes(dw, 1) - all_e
    full_layers = [l for l in range(wl.n_layers) if wl.layer_kinds[l] == ("full" if has_full else "sliding")]
    n_micro_rep = m
    kv_full = sum(dw.algorithmic_kv_bytes(l) for l in full_layers)
    bytes_per_launch = kv_full / len(full_layers) / n_micro_rep
    achieved = bytes_per_launch / (k_ms * 1e-3) / 1e9 if k_ms else None
    traffic, traffic_src = traffic_from_profile(name, wl.batch // m)
    us = ms * 1e3
    gbps = total_b / (ms * 1e-3) / 1e9
    ceiling = probe_ceiling()
    metric = METRIC if wl.n_layers == 36 else METRIC.replace("36-layer decode iteration",
                                                             f"{wl.n_layers}-layer decode step")
    out = {
        "metric": metric, "value": round(us, 1), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.expert_dtype != "e4m3" else "bf16+e4m3",
        "data": "synthetic (seeded generator; GPT-OSS-120B-shaped random weights, no trained checkpoint)",
        "config": {"workload": f"{name}: {wl.n_layers} layers alternating sliding({wl.window})/full, "
                               f"{wl.batch} sequences, KV U[{wl.kv_len_lo},{wl.kv_len_hi}], H {wl.hidden}, "
                               f"{wl.n_q_heads}q/{wl.n_kv_heads}kv x {wl.head_dim}, {wl.n_resident} resident "
                               f"experts of {wl.n_experts} (top-{wl.top_k}), I {wl.inter}"
                               + (f", RoPE base {wl.rope_theta:g}" if wl.rope_theta > 0 else ""),
                   "schedule": sched,
                   "virtual_comm": ({"latency_us": comm[0], "gbps": comm[1],
                                     "endpoints": "attention all-reduce, MoE dispatch, MoE combine per layer"}
                                    if comm else None)},
        "hbm_GBps": round(gbps, 1), "hbm_pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "hbm_probe_ceiling_GBps": ceiling,
        "hbm_pct_probe_ceiling": round(100 * gbps / ceiling, 1) if ceiling else None,
        "algorithmic_GB_per_iter": round(total_b / 1e9, 3),
        "hbm_GBps_min_bytes": round(min_b / (ms * 1e-3) / 1e9, 1),   # the iteration's bytes with weights read once
        "min_GB_per_iter": round(min_b / 1e9, 3),
        "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "per_user_tokens_per_s": round(1 / (ms * 1e-3), 2),
        "schedules_ms": {k: round(v["ms"], 4) for k, v in results.items()},
        "step_ms": results["reported"]["step_ms"],   # per-step spread of the timed steps (host clock)
        "roofline": {"bound": "hbm", "kernel": f"{attn_kernel_name(wl.batch // m, has_full, wl.n_kv_heads, n_cus)} "
                                               f"({'full' if has_full else 'sliding'}-layer decode attention, bf16 KV"
                                               + ("" if has_full else "; the QKV finish folded in: it also reads the "
                                                  "QKV split partials, bytes not counted") + ")",
                     "achieved": round(achieved, 1) if achieved else None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
                     "frac_of_probe_ceiling": round(achieved / ceiling, 4) if achieved and ceiling else None,
                     "traffic": int(traffic) if traffic else None,
                     "bytes_per_launch": int(bytes_per_launch), "mean_launch_ms": k_ms, "launches": k_n,
                     "timer": TIMER_NOTE[args.kernel_timer]},
        "device_error_bits": errs,
        "setup_s": round(t_setup, 1),
    }
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(name)
        except Exception as e:  # the baseline is context, never the product
            out["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
