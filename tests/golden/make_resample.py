"""Writes tests/golden/resample_<workload>.json: for each sequence whose router
margin (gap between the k-th and (k+1)-th fp32 logit) falls below 1e-3 at any
layer, the re-draw index of its initial residual row that clears the margin
at every layer. Only the CPU oracle decides; run on the CPU:

    python tests/golden/make_resample.py gptoss_36l_b64 [more workloads]
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from spatially_pipelined_attention_amd import synth  # noqa: E402
from tests import harness as hz  # noqa: E402


def main(names):
    for name in names:
        wl = synth.WORKLOADS[name]
        t0 = time.time()
        resample, margins = hz.resample_for_margins(wl, list(range(wl.batch)))
        out = {
            "workload": name,
            "seed": wl.seed,
            "margin_min": hz.MARGIN_MIN,
            "resample": {str(k): v for k, v in sorted(resample.items())},
            "min_margin_after": min(margins.values()),
            "generated_by": "tests/golden/make_resample.py (CPU oracle only)",
        }
        path = os.path.join(ROOT, "tests", "golden", f"resample_{name}.json")
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
        print(f"{name}: {len(resample)} re-drawn of {wl.batch}, {time.time() - t0:.0f} s -> {path}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(synth.WORKLOADS))
