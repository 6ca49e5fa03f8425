"""HBM read bandwidth against the CU count of a pool (spa_hbm_probe on CU
pools of 8 .. all CUs, one and two workgroups per CU): the ceiling a stage
kernel on a pool of that size works under, and the device's practical read
ceiling that the benchmark reports its kernels against.

    python -m spatially_pipelined_attention_amd.hbm_probe --command CMD > profiles/hbm_read_probe.md
"""
from __future__ import annotations

import argparse
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=2.0, help="bytes streamed per launch (GiB)")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--command", default="python -m spatially_pipelined_attention_amd.hbm_probe")
    a = ap.parse_args(argv)

    import torch
    from . import binding as B
    ctx = B.spa_init(0)
    n_cus = B.spa_device_cus(ctx)
    counts = sorted({8, 16, 32, 64, 96, 128, 160, 192, 224, n_cus} & set(range(8, n_cus + 1, 8)))
    buf = torch.empty(int(a.gib * (1 << 30)), dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    rows = []
    for n in counts:
        pool = B.spa_pool_create_split(ctx, 0, n)
        try:
            st = B.spa_pool_stream(pool)
            for per_cu in (1, 2):
                wgs = n * per_cu
                nbytes = buf.numel() // (wgs * 1024) * (wgs * 1024)
                ms = B.spa_hbm_probe(ctx, buf, wgs, a.reps, st, nbytes)
                gbps = nbytes / (ms * 1e-3) / 1e9
                rows.append((n, per_cu, ms, gbps))
                print(f"  {n} CUs x {per_cu}: {gbps:.0f} GB/s", file=sys.stderr, flush=True)
        finally:
            B.spa_pool_destroy(pool)
    ceiling = max(r[3] for r in rows if r[0] == n_cus)
    print("# HBM read bandwidth against CU count\n")
    print(f"command: `{a.command}`\n")
    print("spa_hbm_probe on a pool of the first n CUs of every XCD (spa_pool_create_split), "
          f"{a.gib:g} GiB streamed once per launch, mean of {a.reps} launches.\n")
    print(f"- ceiling_GBps: {ceiling:.0f}")
    print(f"- device_cus: {n_cus}")
    print("\n| CUs | workgroups per CU | ms per launch | GB/s | GB/s per CU |")
    print("|---:|---:|---:|---:|---:|")
    for n, pc, ms, g in rows:
        print(f"| {n} | {pc} | {ms:.3f} | {g:.0f} | {g / n:.1f} |")
    B.spa_shutdown(ctx)
    return 0


if __name__ == "__main__":
    sys.exit(main())
