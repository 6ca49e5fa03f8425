"""Text summaries of rocprofv3 output (the files kept under profiles/).

    python -m spatially_pipelined_attention_amd.profiling stats STATS_CSV --command CMD
        kernel table from a `rocprofv3 --kernel-trace --stats --output-format csv` run

    python -m spatially_pipelined_attention_amd.profiling traffic --fetch CSV --write CSV \\
            --kernel NAME --copy-bytes N --command CMD [--sources FILES]
        HBM bytes per launch of one kernel from two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
        runs, scaled by what the same counters read for a plain copy of N bytes in the same
        run (the copy reads N and writes N bytes)

    python -m spatially_pipelined_attention_amd.profiling traffic-table --fetch CSV --write CSV \\
            --kernel PREFIX --copy-bytes N --command CMD
        the same per launch shape of every kernel whose name starts with PREFIX, as a table

    python -m spatially_pipelined_attention_amd.profiling iter-traffic --fetch CSV --write CSV \\
            --copy-bytes N --iterations K --command CMD
        HBM-side bytes of whole iterations: every dispatch of the two counter runs summed per
        kernel name, scaled as above, divided by the K iterations the run executed

    python -m spatially_pipelined_attention_amd.profiling mfma CSV --kernel PREFIX --dtype bf16|f8 \\
            --command CMD
        MFMA work and utilisation per launch of the kernels whose name starts with PREFIX, from a
        `--pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_<DT>` run (MfmaUtil: busy MFMA cycles summed over
        SIMDs over the active cycles of one XCC times the SIMD count)

Each summary is markdown with `key: value` lines that bench.py reads back.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))
# kernels that build a run's inputs rather than run the decode iteration
SETUP_KERNELS = r"k_gen_|k_pack_panels|k_kv_io|FillFunctor|k_fill_i32"


def source_digest(paths: List[str]) -> str:
    h = hashlib.sha256()
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def default_sources(kernel: str) -> List[str]:
    csrc = os.path.join(PKG, "csrc")
    name = "attn.hip" if "attn" in kernel else ("gemm.hip" if "gemm" in kernel else "misc.hip")
    return [os.path.join(csrc, name), os.path.join(csrc, "common.h"), os.path.join(csrc, "kernels.h")]


def read_keys(path: str) -> Dict[str, str]:
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        line = line.strip().lstrip("-").strip()
        if ":" in line and not line.startswith("|"):
            k, v = line.split(":", 1)
            out[k.strip().strip("`")] = v.strip().strip("`")
    return out


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"# Kernel time summary\n\ncommand: `{a.command}`\n")
    print(f"total_kernel_ms: {tot / 1e6:.3f}\n")
    print("| kernel | calls | total ms | mean us | min us | max us | % |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for r in rows[: a.top]:
        print(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
              f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f} |")


def _per_dispatch(path: str) -> List[dict]:
    rows = list(csv.DictReader(open(path)))
    acc = defaultdict(float)
    meta = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        acc[d] += float(r["Counter_Value"])
        meta[d] = (r["Kernel_Name"], int(r["Grid_Size"]))
    return [{"id": d, "name": meta[d][0], "grid": meta[d][1], "kib": acc[d]} for d in sorted(acc)]


def _select(disp: List[dict], kernel: str) -> List[dict]:
    ks = [d for d in disp if d["name"].split("(")[0].replace("void ", "").startswith(kernel)]
    if not ks:
        return []
    gmax = max(d["grid"] for d in ks)   # the largest launch shape of the kernel (full layers)
    return [d for d in ks if d["grid"] == gmax]


def _copy_kib(disp: List[dict]) -> float:
    cs = [d for d in disp if "copy" in d["name"].lower()]
    if not cs:
        raise SystemExit("no copy kernel in the counter file")
    big = max(d["kib"] for d in cs)
    return big


def cmd_traffic(a):
    fetch, write = _per_dispatch(a.fetch), _per_dispatch(a.write)
    kf, kw = _select(fetch, a.kernel), _select(write, a.kernel)
    if not kf or not kw:
        raise SystemExit(f"kernel {a.kernel} not found")
    cf, cw = _copy_kib(fetch), _copy_kib(write)
    f_scale = a.copy_bytes / (cf * 1024.0)
    w_scale = a.copy_bytes / (cw * 1024.0)
    mf = sum(d["kib"] for d in kf) / len(kf)
    mw = sum(d["kib"] for d in kw) / len(kw)
    fetch_b = mf * 1024.0 * f_scale
    write_b = mw * 1024.0 * w_scale
    srcs = a.sources or default_sources(a.kernel)
    print(f"# HBM traffic of `{a.kernel}`\n\ncommand: `{a.command}`\n")
    print(f"- kernel: `{a.kernel}` ({len(kf)} dispatches of grid {kf[0]['grid']})")
    print(f"- copy calibration: {a.copy_bytes} bytes read and written; FETCH_SIZE {cf:.0f} KiB, "
          f"WRITE_SIZE {cw:.0f} KiB -> scale fetch {f_scale:.4f}, write {w_scale:.4f}")
    print(f"- mean FETCH_SIZE {mf:.0f} KiB, WRITE_SIZE {mw:.0f} KiB per dispatch")
    print(f"- fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"- write_bytes_per_launch: {write_b:.0f}")
    print(f"- traffic_bytes_per_launch: {fetch_b + write_b:.0f}")
    print(f"- kernel_source_digest: {source_digest(srcs)}")
    print(f"- kernel_sources: {', '.join(os.path.relpath(p, os.path.dirname(PKG)) for p in srcs)}")
    for kv in a.set or []:
        k, v = kv.split("=", 1)
        print(f"- {k}: {v}")


def cmd_iter_traffic(a):
    fetch, write = _per_dispatch(a.fetch), _per_dispatch(a.write)
    f_scale = a.copy_bytes / (_copy_kib(fetch) * 1024.0)
    w_scale = a.copy_bytes / (_copy_kib(write) * 1024.0)

    skip = re.compile(a.exclude)

    def sums(disp, sc):
        g = defaultdict(lambda: [0, 0.0])
        for d in disp:
            name = d["name"].split("(")[0].replace("void ", "")
            if "copy" in name.lower() or name.startswith("__amd") or skip.search(name):
                continue
            g[name][0] += 1
            g[name][1] += d["kib"] * 1024.0 * sc
        return g

    gf, gw = sums(fetch, f_scale), sums(write, w_scale)
    K = a.iterations
    tf = sum(v[1] for v in gf.values()) / K
    tw = sum(v[1] for v in gw.values()) / K
    print(f"# HBM-side traffic per iteration\n\ncommand: `{a.command}`\n")
    print(f"Counter scale from a plain copy of {a.copy_bytes} bytes: fetch x{f_scale:.4f}, write x{w_scale:.4f}. "
          f"Every dispatch of the run except the copies, runtime helpers and the input set-up kernels "
          f"(`{a.exclude}`), divided by {K} iterations.\n")
    print(f"- fetch_GB_per_iter: {tf / 1e9:.3f}")
    print(f"- write_GB_per_iter: {tw / 1e9:.3f}")
    print(f"- traffic_GB_per_iter: {(tf + tw) / 1e9:.3f}")
    for kv in a.set or []:
        k, v = kv.split("=", 1)
        print(f"- {k}: {v}")
    print("\n| kernel | launches per iteration | fetch MB per iteration | write MB per iteration |")
    print("|---|---:|---:|---:|")
    for name in sorted(gf, key=lambda n: -gf[n][1]):
        print(f"| `{name}` | {gf[name][0] / K:.0f} | {gf[name][1] / K / 1e6:.1f} | {gw.get(name, [0, 0.0])[1] / K / 1e6:.1f} |")


def cmd_traffic_table(a):
    fetch, write = _per_dispatch(a.fetch), _per_dispatch(a.write)
    f_scale = a.copy_bytes / (_copy_kib(fetch) * 1024.0)
    w_scale = a.copy_bytes / (_copy_kib(write) * 1024.0)

    def groups(disp, sc):
        g = defaultdict(list)
        for d in disp:
            name = d["name"].split("(")[0].replace("void ", "")
            if name.startswith(a.kernel):
                g[(name, d["grid"])].append(d["kib"] * 1024.0 * sc)
        return g

    gf, gw = groups(fetch, f_scale), groups(write, w_scale)
    print(f"# HBM traffic per launch of `{a.kernel}*`\n\ncommand: `{a.command}`\n")
    print(f"Counter scale from a plain copy of {a.copy_bytes} bytes: fetch x{f_scale:.4f}, write x{w_scale:.4f}.\n")
    print("| kernel | grid | launches | fetch MB | write MB |")
    print("|---|---:|---:|---:|---:|")
    for key in sorted(gf, key=lambda k: -sum(gf[k])):
        f = gf[key]
        w = gw.get(key, [0.0])
        print(f"| `{key[0]}` | {key[1]} | {len(f)} | {sum(f) / len(f) / 1e6:.2f} | {sum(w) / len(w) / 1e6:.2f} |")


PEAK_TFLOPS = {"bf16": 2500.0, "f8": 5000.0}   # dense MFMA peaks of the device


def cmd_mfma(a):
    rows = list(csv.DictReader(open(a.csv)))
    per = defaultdict(dict)
    meta = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        meta[d] = (r["Kernel_Name"].split("(")[0].replace("void ", ""), int(r["Grid_Size"]),
                   (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    mops = f"SQ_INSTS_VALU_MFMA_MOPS_{a.dtype.upper()}"
    groups = defaultdict(list)
    for d, c in per.items():
        name, grid, dur = meta[d]
        if name.startswith(a.kernel) and mops in c and "MfmaUtil" in c:
            groups[(name, grid)].append((c[mops] * 512.0, c["MfmaUtil"], dur))
    if not groups:
        raise SystemExit(f"no launch of {a.kernel} with {mops} and MfmaUtil")
    print(f"# MFMA work of `{a.kernel}*` ({a.dtype})\n\ncommand: `{a.command}`\n")
    print(f"Dense {a.dtype} MFMA peak: {PEAK_TFLOPS[a.dtype]:.0f} TFLOP/s. Durations are those of the counter run "
          "(launches serialised by the profiler).\n")
    print("| kernel | grid | launches | mean us | GFLOP per launch | TFLOP/s | % of peak | MfmaUtil % |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        n = len(v)
        fl = sum(x[0] for x in v) / n
        ut = sum(x[1] for x in v) / n
        du = sum(x[2] for x in v) / n
        tf = fl / du / 1e12
        print(f"| `{name}` | {grid} | {n} | {du * 1e6:.2f} | {fl / 1e9:.3f} | {tf:.1f} | "
              f"{100 * tf / PEAK_TFLOPS[a.dtype]:.1f} | {ut:.1f} |")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=25)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--sources", nargs="*")
    t.add_argument("--set", action="append", metavar="KEY=VALUE", help="extra key recorded in the summary")
    it = sub.add_parser("iter-traffic")
    it.add_argument("--fetch", required=True)
    it.add_argument("--write", required=True)
    it.add_argument("--copy-bytes", type=int, required=True)
    it.add_argument("--iterations", type=int, required=True)
    it.add_argument("--command", required=True)
    it.add_argument("--set", action="append")
    it.add_argument("--exclude", default=SETUP_KERNELS,
                    help="regex of kernel names that build the inputs (generator, weight packing, KV writes, fills)")
    tt = sub.add_parser("traffic-table")
    tt.add_argument("--fetch", required=True)
    tt.add_argument("--write", required=True)
    tt.add_argument("--kernel", required=True)
    tt.add_argument("--copy-bytes", type=int, required=True)
    tt.add_argument("--command", required=True)
    mf = sub.add_parser("mfma")
    mf.add_argument("csv")
    mf.add_argument("--kernel", required=True)
    mf.add_argument("--dtype", choices=["bf16", "f8"], required=True)
    mf.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "iter-traffic": cmd_iter_traffic, "traffic-table": cmd_traffic_table,
     "mfma": cmd_mfma}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
