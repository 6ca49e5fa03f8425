"""The SubGPU execution model's timing and search pieces, in plain Python.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows section 3 of the SubGPU Pipelining paper: the segment-to-stage
binding (equation 1), the augmented task DAG of section 3.2 and its max-plus
recurrence (equations 4-5), the configuration count of section 3.3
(equation 7), and the pairwise-line SM-allocation refinement of section 4.2
(Algorithm 2), each written from the text, not from a listing.
"""
from __future__ import annotations

import itertools
import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

Task = Tuple[int, int, int]   # (region instance l, microbatch mu, segment k), k is 1-based


def binding(k: int, K: int, w: int) -> int:
    """Equation 1: segment k of K runs on stage 1 when boundary reuse is on
    (w = 1) and k is the last segment; otherwise on stage k."""
    return 1 if (w == 1 and k == K) else k


def tasks_in_dispatch_order(n_regions: int, m: int, K: int) -> List[Task]:
    """Segment tasks (l, mu, k) in the fixed global dispatch order.

    Section 3.2 asks for a topological order of the data dependencies; the
    reading taken is region-major, then microbatch, then segment, which is
    topological because every data edge goes to a larger (l, mu, k) key.
    """
    return [(l, mu, k) for l in range(n_regions) for mu in range(m) for k in range(1, K + 1)]


def data_predecessors(t: Task, K: int) -> List[Task]:
    """A segment consumes the previous segment of the same microbatch; the
    first segment of region l consumes the last segment of region l-1."""
    l, mu, k = t
    if k > 1:
        return [(l, mu, k - 1)]
    if l > 0:
        return [(l - 1, mu, K)]
    return []


def makespan(n_regions: int, m: int, K: int, w: int, tau: Callable[[Task], float],
             order: Optional[Sequence[Task]] = None):
    """Equations 4-5: A_i = max(max over data preds C_j, max over stage preds C_j),
    C_i = A_i + tau_i, T = max_i C_i (empty maxima are zero). Stage predecessor
    = the previous task on the same stage in the global order. Returns
    (T, {task: (A, C)})."""
    order = list(order) if order is not None else tasks_in_dispatch_order(n_regions, m, K)
    pos = {t: i for i, t in enumerate(order)}
    last_on_stage: Dict[int, Task] = {}
    times: Dict[Task, Tuple[float, float]] = {}
    for t in order:
        start = 0.0
        for p in data_predecessors(t, K):
            if pos[p] >= pos[t]:
                raise ValueError("dispatch order is not topological")
            start = max(start, times[p][1])
        st = binding(t[2], K, w)
        if st in last_on_stage:
            start = max(start, times[last_on_stage[st]][1])
        times[t] = (start, start + float(tau(t)))
        last_on_stage[st] = t
    T = max((c for _, c in times.values()), default=0.0)
    return T, times


def augmented_edges(n_regions: int, m: int, K: int, w: int, order: Optional[Sequence[Task]] = None):
    """All edges (data and stage) of the augmented task DAG, for cross-checks."""
    order = list(order) if order is not None else tasks_in_dispatch_order(n_regions, m, K)
    edges = []
    last: Dict[int, Task] = {}
    for t in order:
        for p in data_predecessors(t, K):
            edges.append((p, t))
        st = binding(t[2], K, w)
        if st in last:
            edges.append((last[st], t))
        last[st] = t
    return order, edges


# --------------------------------------------------------------------------
# search-space size (section 3.3, equation 7)
# --------------------------------------------------------------------------
def chain_cuts(n_ops: int, n_segments: int) -> int:
    """|C_K(G)| for a chain of n_ops operators: ways to cut it into K nonempty
    contiguous segments (choose K-1 of the n_ops-1 gaps)."""
    if n_segments < 1 or n_segments > n_ops:
        return 0
    return math.comb(n_ops - 1, n_segments - 1)


def cut_and_binding_choices(n_ops: int, n_stages: int) -> int:
    """One-to-one (K = D) plus boundary-reuse (K = D + 1) cut sets."""
    return chain_cuts(n_ops, n_stages) + chain_cuts(n_ops, n_stages + 1)


def allocations(n_units: int, n_stages: int, quantum: int, p_min: Optional[int] = None) -> int:
    """Ordered allocations of n_units to n_stages, each a positive multiple of
    the quantum (at least p_min), using the whole budget: brute-force count."""
    p_min = quantum if p_min is None else p_min
    q = n_units // quantum
    lo = -(-p_min // quantum)
    cnt = 0

    def rec(stages_left, quanta_left):
        nonlocal cnt
        if stages_left == 1:
            if quanta_left >= lo:
                cnt += 1
            return
        for a in range(lo, quanta_left - lo * (stages_left - 1) + 1):
            rec(stages_left - 1, quanta_left - a)

    if n_units % quantum == 0:
        rec(n_stages, q)
    return cnt


# --------------------------------------------------------------------------
# pairwise-line allocation refinement (section 4.2, Algorithm 2)
# --------------------------------------------------------------------------
def pairwise_line(f: Callable[[Tuple[int, ...]], float], feasible: Callable[[Tuple[int, ...]], bool],
                  p0: Sequence[int], quantum: int, pass_limit: Optional[int] = None):
    """Refine an allocation by moving quanta between one donor and one receiver stage.

    Each pass: among all legal one-quantum moves (donor d -> receiver r) take
    the one with the smallest objective (ties: lowest (d, r)). Stop if it does
    not improve on the current value. Otherwise search along that line: keep a
    step h (starting at 1) and the best move size z; try z + h, doubling h on
    improvement and halving it (integer) otherwise, until h reaches zero; apply
    the best z. Repeat until no improving move or the pass limit.
    Returns (p, f(p), number of objective evaluations).
    """
    p = tuple(p0)
    evals = 0

    def F(x):
        nonlocal evals
        evals += 1
        return f(x)

    def move(x, d, r, z):
        y = list(x)
        y[d] -= z * quantum
        y[r] += z * quantum
        return tuple(y)

    t = F(p)
    n = len(p)
    passes = 0
    while pass_limit is None or passes < pass_limit:
        passes += 1
        cands = [(d, r) for d in range(n) for r in range(n) if d != r and feasible(move(p, d, r, 1))]
        if not cands:
            return p, t, evals
        vals = [(F(move(p, d, r, 1)), d, r) for d, r in cands]
        best = min(vals)
        t_line, d, r = best
        if t_line >= t:
            return p, t, evals
        z, h = 1, 1
        while h > 0:
            zz = z + h
            cand = move(p, d, r, zz)
            if feasible(cand):
                v = F(cand)
                if v < t_line:
                    z, t_line, h = zz, v, 2 * h
                    continue
            h //= 2
        p, t = move(p, d, r, z), t_line
    return p, t, evals
