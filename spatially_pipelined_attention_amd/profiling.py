"""Text summaries of rocprofv3 output (the files kept under profiles/).

    python -m spatially_pipelined_attention_amd.profiling stats STATS_CSV --command CMD
        kernel table from a `rocprofv3 --kernel-trace --stats --output-format csv` run

    python -m spatially_pipelined_attention_amd.profiling traffic --fetch CSV --write CSV \\
            --kernel NAME --copy-bytes N --command CMD [--sources FILES]
        HBM bytes per launch of one kernel from two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
        runs, scaled by what the same counters read for a plain copy of N bytes in the same
        run (the copy reads N and writes N bytes)

Each summary is markdown with `key: value` lines that bench.py reads back.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import sys
from collections import defaultdict
from typing import Dict, List

PKG = os.path.dirname(os.path.abspath(__file__))


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
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
