"""The SubGPU execution model's timing and search pieces, in plain Python.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows section 3 of the SubGPU Pipelining paper: the segment-to-stage
binding (equation 1), the augmented task DAG of section 3.2 and its max-plus
recurrence (equations 4-5), the configuration count of section 3.3
(equation 7), and the pairwise-line SM-allocation refinement of section 4.2
(Algorithm 2); the refinement follows the section's prose description of
the method, in this module's own structure.
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
# pairwise-line allocation refinement (section 4.2)
# --------------------------------------------------------------------------
def _shift(p: Tuple[int, ...], donor: int, receiver: int, amount: int) -> Tuple[int, ...]:
    """p with `amount` CUs taken from the donor stage and given to the receiver."""
    y = list(p)
    y[donor] -= amount
    y[receiver] += amount
    return tuple(y)


def _gallop(value_at: Callable[[int], Optional[float]], z: int, best: float) -> Tuple[int, float]:
    """One-dimensional search over a transfer size z >= 1 (in quanta), starting
    from a size already known to give `best`. A trial at z + step that
    improves is taken and the step doubles; any other trial (worse, or
    illegal: value_at returns None) halves the step; the search ends when the
    step reaches zero."""
    step = 1
    while step:
        v = value_at(z + step)
        if v is not None and v < best:
            z, best, step = z + step, v, step * 2
        else:
            step //= 2
    return z, best


def pairwise_line(f: Callable[[Tuple[int, ...]], float], feasible: Callable[[Tuple[int, ...]], bool],
                  p0: Sequence[int], quantum: int, pass_limit: Optional[int] = None):
    """Section 4.2's allocation refinement: local search over CU allocations by
    pairwise transfers between stages.

    A pass looks at every ordered (donor, receiver) pair whose one-quantum
    transfer stays legal and ranks the pairs by the objective after that
    transfer (ties to the lowest pair). If the best of them is no better than
    the current allocation, the search has converged. Otherwise the pass
    follows that pair's line: larger transfers along the same direction are
    tried with a doubling/halving step (_gallop) and the best one is applied.
    The search stops when no legal pairwise move improves the objective or
    after pass_limit passes. Returns (p, f(p), objective evaluations).
    """
    n_eval = 0

    def cost(x):
        nonlocal n_eval
        n_eval += 1
        return f(x)

    p = tuple(p0)
    current = cost(p)
    passes = 0
    while pass_limit is None or passes < pass_limit:
        passes += 1
        probes = []
        for d in range(len(p)):
            for r in range(len(p)):
                if d != r and feasible(_shift(p, d, r, quantum)):
                    probes.append((cost(_shift(p, d, r, quantum)), d, r))
        if not probes:
            break
        v1, d, r = min(probes)
        if v1 >= current:
            break

        def along(z, _d=d, _r=r):
            cand = _shift(p, _d, _r, z * quantum)
            return cost(cand) if feasible(cand) else None

        z, current = _gallop(along, 1, v1)
        p = _shift(p, d, r, z * quantum)
    return p, current, n_eval
