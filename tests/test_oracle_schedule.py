"""Pins of the oracle's execution-model pieces (CPU): the page's printed
search-space counts, closed forms of the max-plus recurrence, an independent
longest-path routine, and brute-force optima for the allocation refinement."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import shortest_path

from oracle import schedule as os_

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "subgpu_search_space.json")


def test_search_space_counts_match_page():
    g = json.load(open(GOLDEN))
    c = g["cut_and_binding"]
    assert os_.cut_and_binding_choices(c["n_ops"], c["n_stages"]) == c["value"]
    a = g["allocations"]
    assert os_.allocations(a["n_sm"], a["n_stages"], a["quantum"]) == a["value"]
    prod = c["value"] * a["value"]
    assert abs(prod / g["product_order_of_magnitude"]["value"] - 1) < 0.05


def test_binding_equation_1():
    assert [os_.binding(k, 5, 0) for k in range(1, 6)] == [1, 2, 3, 4, 5]
    assert [os_.binding(k, 6, 1) for k in range(1, 7)] == [1, 2, 3, 4, 5, 1]


@pytest.mark.parametrize("tA,tB,m", [(3.0, 5.0, 1), (3.0, 5.0, 4), (7.0, 2.0, 6), (4.0, 4.0, 3)])
def test_two_stage_one_region_closed_form(tA, tB, m):
    T, _ = os_.makespan(1, m, 2, 0, lambda t: tA if t[2] == 1 else tB)
    assert T == pytest.approx(tA + tB + (m - 1) * max(tA, tB))


def test_steady_state_rate_is_one_over_slower_stage():
    # throughput of a balanced-or-not two-stage pipeline tends to 1/max(t1, t2)
    for tA, tB in ((2.0, 5.0), (6.0, 1.5)):
        T1, _ = os_.makespan(1, 1000, 2, 0, lambda t: tA if t[2] == 1 else tB)
        T2, _ = os_.makespan(1, 2000, 2, 0, lambda t: tA if t[2] == 1 else tB)
        assert (T2 - T1) / 1000 == pytest.approx(max(tA, tB))


def test_temporal_is_one_stage_sum():
    # K = D = 1: every task serialises on the single stage
    rng = np.random.default_rng(0)
    taus = {}
    T, _ = os_.makespan(3, 2, 1, 0, lambda t: taus.setdefault(t, float(rng.uniform(1, 3))))
    assert T == pytest.approx(sum(taus.values()))


@pytest.mark.parametrize("n_regions,m,K,w", [(1, 3, 2, 0), (3, 2, 2, 0), (4, 4, 3, 1), (2, 5, 3, 0), (3, 1, 4, 1)])
def test_makespan_equals_longest_path(n_regions, m, K, w):
    rng = np.random.default_rng(n_regions * 100 + m * 10 + K)
    taus = {}
    tau = lambda t: taus.setdefault(t, float(rng.uniform(0.5, 4.0)))
    T, _ = os_.makespan(n_regions, m, K, w, tau)
    order, edges = os_.augmented_edges(n_regions, m, K, w)
    # longest path: node-weighted DAG -> edge weights; source/sink added; negate for shortest path
    idx = {t: i + 1 for i, t in enumerate(order)}
    N = len(order) + 2
    rows, cols, vals = [], [], []
    for t in order:
        rows.append(0); cols.append(idx[t]); vals.append(-1e-300)           # source
        rows.append(idx[t]); cols.append(N - 1); vals.append(-tau(t))       # sink
    for a, b in sorted(set(edges)):       # a data edge may coincide with a stage edge
        rows.append(idx[a]); cols.append(idx[b]); vals.append(-tau(a))
    G = csr_matrix((vals, (rows, cols)), shape=(N, N))
    d = shortest_path(G, method="BF", directed=True, indices=0)
    assert -d[N - 1] == pytest.approx(T, rel=1e-12)


def test_non_topological_order_rejected():
    order = os_.tasks_in_dispatch_order(1, 2, 2)
    bad = [order[1], order[0]] + order[2:]
    with pytest.raises(ValueError):
        os_.makespan(1, 2, 2, 0, lambda t: 1.0, order=bad)


def _brute_best(f, total, n, quantum, pmin):
    best = None
    q = total // quantum
    for parts in itertools.product(range(pmin // quantum, q + 1), repeat=n - 1):
        last = q - sum(parts)
        if last < pmin // quantum:
            continue
        p = tuple(x * quantum for x in parts) + (last * quantum,)
        v = f(p)
        if best is None or v < best[0]:
            best = (v, p)
    return best


@pytest.mark.parametrize("n,total,quantum,seed", [(2, 256, 8, 0), (2, 256, 8, 1), (3, 96, 4, 2), (3, 120, 8, 3)])
def test_pairwise_line_reaches_brute_force_optimum_on_balanced_stages(n, total, quantum, seed):
    # stage time = work_d / p_d (a pipeline's slowest stage sets the rate): the
    # max over stages is quasi-convex in the transfer along any donor/receiver line
    rng = np.random.default_rng(seed)
    work = rng.uniform(1, 10, n)
    f = lambda p: float(max(work[d] / p[d] for d in range(n)))
    feasible = lambda p: all(x >= quantum for x in p) and sum(p) == total
    p0 = tuple([total // n // quantum * quantum] * (n - 1) + [total - (n - 1) * (total // n // quantum * quantum)])
    p, t, _ = os_.pairwise_line(f, feasible, p0, quantum)
    best, _ = _brute_best(f, total, n, quantum, quantum)
    assert t == pytest.approx(best)


def test_pairwise_line_stops_without_improving_move_and_respects_pass_limit():
    f = lambda p: abs(p[0] - 64)
    feasible = lambda p: min(p) >= 8 and sum(p) == 128
    p, t, ev = os_.pairwise_line(f, feasible, (64, 64), 8)
    assert p == (64, 64) and t == 0 and ev == 3        # f(p0) + the two one-quantum moves
    p, t, _ = os_.pairwise_line(lambda p: -p[0], feasible, (64, 64), 8, pass_limit=1)
    assert p == (120, 8)                               # one line search runs to the boundary
