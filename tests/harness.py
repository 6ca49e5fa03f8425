"""Test-side glue: runs the CPU oracle on generator inputs for chosen tokens,
and compares results with the bars used throughout the tests."""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle import layer as ol
from spatially_pipelined_attention_amd import synth

MARGIN_MIN = 1e-3

# max |err| <= TOL * RMS(reference): bf16 and fp8 bars as stated for the
# workloads; fp32 from the arithmetic (fp32 accumulation over <= 4096 terms,
# typical relative error sqrt(K) * 2^-24 ~ 4e-6, bounded by K * 2^-24 ~ 2.4e-4)
TOL = {"bf16": 2e-2, "e4m3": 6e-2, "f32": 2.5e-4}


def dims(wl: synth.Workload) -> ol.Dims:
    return ol.Dims(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_experts, wl.n_resident, wl.top_k,
                   wl.inter, wl.window, wl.eps, wl.rope_theta)


def numerics(wl: synth.Workload) -> ol.Numerics:
    act = "bf16" if wl.w_dtype == "bf16" else "none"
    kv = "bf16" if wl.kv_dtype == "bf16" else "none"
    ex = {"bf16": "bf16", "e4m3": "e4m3", "f32": "none"}[wl.expert_dtype]
    return ol.Numerics(act, kv, ex)


def tol_of(wl: synth.Workload) -> float:
    return TOL["e4m3"] if wl.expert_dtype == "e4m3" else TOL[wl.w_dtype]


def layer_params(wl: synth.Workload, l: int):
    dense = synth.dense_weights(wl, l)
    return dense, (lambda e: synth.expert_weights(wl, l, e))


def run_oracle(wl: synth.Workload, tokens: Sequence[int], resample: Optional[Dict[int, int]] = None,
               n_layers: Optional[int] = None, keep_records: bool = False, progress: bool = True):
    """Oracle decode iteration for the given sequences (any subset: tokens are independent)."""
    tokens = list(tokens)
    L = synth.kv_lengths(wl)[tokens]
    x = synth.x_rows(wl, tokens, resample)
    kinds = wl.layer_kinds[: (n_layers or wl.n_layers)]

    def history(l, bi, lo, hi):
        return synth.kv_history(wl, l, tokens[bi], lo, hi)

    def params(l):
        if progress:
            print(f"  oracle layer {l} ({len(tokens)} sequences)", flush=True)
        return layer_params(wl, l)

    return ol.iteration_forward(dims(wl), numerics(wl), kinds, x, params, L, history, keep_records)


def resample_for_margins(wl: synth.Workload, tokens: Sequence[int], max_rounds: int = 12,
                         n_layers: Optional[int] = None):
    """Re-draw x of any token whose router margin falls below 1e-3 at some
    layer, until every token clears it. Returns (resample map, final margins)."""
    resample: Dict[int, int] = {}
    pending = list(tokens)
    margins: Dict[int, float] = {}
    for _ in range(max_rounds):
        if not pending:
            break
        _, _, mg, _ = run_oracle(wl, pending, resample, n_layers)
        low = []
        for i, b in enumerate(pending):
            mmin = float(np.min(mg[:, i]))
            margins[b] = mmin
            if mmin < MARGIN_MIN:
                resample[b] = resample.get(b, 0) + 1
                low.append(b)
        pending = low
    if pending:
        raise RuntimeError(f"tokens {pending} keep router margins below {MARGIN_MIN}")
    return resample, margins


def assert_close_rms(got, ref, tol: float, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol * rms, f"{what}: max|err| {err:.3e} > {tol} * RMS {rms:.3e}"
    return err / max(rms, 1e-300)


def load_resample(name: str) -> Dict[int, int]:
    """Re-draw map stored by tests/golden/make_resample.py (empty if absent)."""
    import json
    import os
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", f"resample_{name}.json")
    if not os.path.exists(p):
        return {}
    return {int(k): int(v) for k, v in json.load(open(p))["resample"].items()}
