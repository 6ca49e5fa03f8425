"""Host logic of the throughput-frontier sweep (no GPU)."""
from spatially_pipelined_attention_amd.pareto import frontier


def _pt(u, g, tag):
    return {"per_user": u, "per_gpu": g, "tag": tag}


def test_frontier_keeps_only_undominated_points_sorted_by_per_user():
    pts = [_pt(10, 100, "a"), _pt(20, 80, "b"), _pt(15, 70, "c"), _pt(5, 120, "d"), _pt(20, 60, "e")]
    f = frontier(pts)
    assert [p["tag"] for p in f] == ["d", "a", "b"]   # c is beaten by b, e by b


def test_frontier_keeps_exact_duplicates_and_single_points():
    assert [p["tag"] for p in frontier([_pt(1, 1, "x")])] == ["x"]
    f = frontier([_pt(3, 3, "p"), _pt(3, 3, "q")])
    assert sorted(p["tag"] for p in f) == ["p", "q"]
