"""The C-ABI library on the CPU: loads, exports every declared symbol, and its
host-only entry points (validation, workspace sizing, schedule model,
allocation refinement) agree with the oracle and the page's printed counts.
No kernel is launched here."""
import ctypes as C
import itertools
import json
import os
import re

import numpy as np
import pytest

from oracle import schedule as osch
from spatially_pipelined_attention_amd import binding as B
from spatially_pipelined_attention_amd import synth
from spatially_pipelined_attention_amd.workload import model_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(spa_[a-z0-9_]+)\s*\(", txt))
    # typedef'd function pointer type is not a symbol
    names.discard("spa_objective_fn")
    return names


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    decl = declared_symbols()
    assert len(decl) >= 30
    missing = [n for n in sorted(decl) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(B.EXPORTED) == decl


def test_init_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(B.SpaError):
        B.spa_init(0)
    assert B.spa_last_error()


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_query_accepts_every_workload(name):
    wl = synth.WORKLOADS[name]
    m = model_desc(wl)
    for n_micro in (1, 2, 4):
        if wl.batch % n_micro:
            continue
        nb = B.spa_workspace_query(m, wl.batch, wl.kv_len_hi, n_micro)
        assert nb > 0
    # more microbatches of the same batch never need less than one
    assert B.spa_workspace_query(m, wl.batch, wl.kv_len_hi, 1) > 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 128, B.SPA_EUNSUPPORTED),
    ("n_q_heads", 63, B.SPA_EINVAL),
    ("hidden", 2881, B.SPA_EINVAL),
    ("inter", 2881, B.SPA_EINVAL),
    ("window", 100, B.SPA_EINVAL),
    ("top_k", 0, B.SPA_EINVAL),
    ("top_k", 9, B.SPA_EINVAL),
    ("n_resident", 0, B.SPA_EINVAL),
    ("n_experts", 300, B.SPA_EUNSUPPORTED),
    ("kv_dtype", B.SPA_F32, B.SPA_EUNSUPPORTED),
    ("expert_dtype", 7, B.SPA_EINVAL),
])
def test_model_validation_errors(field, value, status):
    m = model_desc(synth.WORKLOADS["gptoss_layer_full"])
    setattr(m, field, value)
    with pytest.raises(B.SpaError) as ei:
        B.spa_workspace_query(m, 64, 4096, 1)
    assert ei.value.status == status


@pytest.mark.parametrize("latency,gbps", [(-1.0, 900.0), (2000.0, 900.0), (float("nan"), 900.0), (3.0, -1.0),
                                           (3.0, 2e5), (3.0, float("nan"))])
def test_comm_model_validation(latency, gbps):
    m = model_desc(synth.WORKLOADS["gptoss_36l_b64"])
    m.comm_latency_us, m.comm_gbps = latency, gbps
    with pytest.raises(B.SpaError) as ei:
        B.spa_workspace_query(m, 64, 8192, 1)
    assert ei.value.status == B.SPA_EINVAL


@pytest.mark.parametrize("name,n_micro", [("gptoss_36l_b64", 1), ("gptoss_36l_b64", 4), ("gptoss_36l_fp8", 2),
                                          ("tiny_fp32", 1)])
def test_comm_receive_buffer_is_the_largest_payload(name, n_micro):
    """With endpoints, every microbatch slot holds one receive buffer as large
    as the largest of the layer's three payloads: b*H dense values (all-reduce),
    b*k*H expert-input values plus E4M3 row scales (dispatch), b*k*H dense
    values (combine), b = tokens per microbatch; rounded up to 256 bytes."""
    wl = synth.WORKLOADS[name]
    m = model_desc(wl)
    base = B.spa_workspace_query(m, wl.batch, wl.kv_len_hi, n_micro)
    m.comm_latency_us, m.comm_gbps = 3.0, 900.0
    with_comm = B.spa_workspace_query(m, wl.batch, wl.kv_len_hi, n_micro)
    esz = {"f32": 4, "bf16": 2, "e4m3": 1}
    b = wl.batch // n_micro
    dn, ex = esz[wl.w_dtype], esz[wl.expert_dtype]
    payload = max(b * wl.hidden * dn, b * wl.top_k * wl.hidden * ex + (b * wl.top_k * 4 if ex == 1 else 0),
                  b * wl.top_k * wl.hidden * dn)
    assert with_comm - base == n_micro * ((payload + 255) // 256 * 256)


def test_microbatch_must_divide_batch():
    m = model_desc(synth.WORKLOADS["gptoss_36l_b64"])
    with pytest.raises(B.SpaError) as ei:
        B.spa_workspace_query(m, 64, 8192, 3)
    assert ei.value.status == B.SPA_EINVAL


def test_sched_binding_matches_oracle():
    for K in range(2, 7):
        for w in (0, 1):
            for k in range(1, K + 1):
                assert B.spa_sched_binding(k, K, w) == osch.binding(k, K, w)


@pytest.mark.parametrize("n_regions,m,K,w", [(1, 4, 2, 0), (36, 2, 2, 0), (36, 4, 2, 0), (6, 3, 3, 1), (2, 8, 5, 1)])
def test_sched_makespan_matches_oracle(n_regions, m, K, w):
    rng = np.random.default_rng(n_regions * 31 + m)
    tau = rng.uniform(0.1, 5.0, n_regions * m * K)
    T, st, en = B.spa_sched_makespan(n_regions, m, K, w, tau)
    ref, times = osch.makespan(n_regions, m, K, w, lambda t: tau[(t[0] * m + t[1]) * K + t[2] - 1])
    assert T == pytest.approx(ref, rel=1e-12)
    for (l, mu, k), (a, c) in times.items():
        i = (l * m + mu) * K + k - 1
        assert st[i] == pytest.approx(a, rel=1e-12, abs=1e-12)
        assert en[i] == pytest.approx(c, rel=1e-12)


def test_sched_counts_match_page_and_oracle():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "subgpu_search_space.json")))
    cuts, allocs = B.spa_sched_counts(g["cut_and_binding"]["n_ops"], g["cut_and_binding"]["n_stages"],
                                      g["allocations"]["n_sm"], g["allocations"]["quantum"])
    assert cuts == g["cut_and_binding"]["value"]
    assert allocs == g["allocations"]["value"]
    for n_ops, D, N, q in ((7, 2, 256, 8), (10, 3, 64, 4), (5, 4, 32, 2)):
        c, a = B.spa_sched_counts(n_ops, D, N, q)
        assert c == osch.cut_and_binding_choices(n_ops, D)
        assert a == osch.allocations(N, D, q)


@pytest.mark.parametrize("n,total,quantum,seed", [(2, 256, 8, 0), (2, 256, 8, 5), (3, 96, 4, 2), (4, 128, 8, 3)])
def test_refine_allocation_matches_oracle(n, total, quantum, seed):
    rng = np.random.default_rng(seed)
    work = rng.uniform(1, 10, n)
    noise = rng.uniform(0, 0.05, 10000)

    def f(p):
        # stage-time model with a deterministic bump so ties and plateaus occur
        return float(max(work[d] / p[d] for d in range(len(p))) + noise[hash(p) % 10000] * 0)

    feasible = lambda p: all(v >= quantum and v % quantum == 0 for v in p) and sum(p) == total
    base = total // n // quantum * quantum
    p0 = tuple([base] * (n - 1) + [total - base * (n - 1)])
    ref_p, ref_t, ref_ev = osch.pairwise_line(f, feasible, p0, quantum)
    p, t, ev = B.spa_refine_allocation(n, total, quantum, quantum, p0, f)
    assert p == ref_p and t == pytest.approx(ref_t) and ev == ref_ev


def test_refine_allocation_pass_limit_and_infeasible_start():
    p, t, ev = B.spa_refine_allocation(2, 128, 8, 8, (64, 64), lambda p: -p[0], pass_limit=1)
    assert p == (120, 8)
    with pytest.raises(B.SpaError):
        B.spa_refine_allocation(2, 128, 8, 8, (60, 68), lambda p: 0.0)
