"""Routing in one launch, on the GPU, through the C ABI (spa_moe_route): top-k
of the router logits and the dispatch permutation, which the last top-k
workgroup to finish computes.

Calls of different token counts run one after another on one workspace, so
each call must find the arrival counter cleared by the call before: odd
counts (a workgroup holding one token), a single token, more workgroups than
the device holds at once, and the largest call (1,024 tokens, 4,096 picks
over 128 resident experts: the permutation's largest LDS). The picks are
checked against the rule applied to the GPU's own logits (the larger logit
first, equal logits to the lower index), the weights against the softmax over
the picks, and the permutation bit for bit against the oracle's permutation
of the GPU's picks.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_one_launch_routing_over_calls_of_several_sizes():
    from oracle.layer import permutation
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    wl = synth.WORKLOADS["gptoss_layer_full"]   # 128 resident experts, top-4
    print("\n[route] building gptoss_layer_full", flush=True)
    dw = DeviceWorkload(wl)
    ctx = B.spa_init(0)
    m, lay = dw.m, dw.layers_c[0]
    H, E, k, Er = wl.hidden, wl.n_experts, wl.top_k, wl.n_resident
    nmax = 1024
    ws = dw.workspace(n_tok=nmax)
    gen = torch.Generator(device="cuda").manual_seed(11)
    hn_all = torch.randn(nmax, H, device="cuda", generator=gen)
    for n in (7, 1, 64, 129, nmax, 33):
        print(f"[route] {n} tokens", flush=True)
        hn = hn_all[:n].contiguous()
        logits = torch.zeros(n, E, device="cuda")
        idx = torch.full((n, k), -1, dtype=torch.int32, device="cuda")
        w = torch.zeros(n, k, device="cuda")
        offs = torch.full((Er + 1,), -1, dtype=torch.int32, device="cuda")
        rt = torch.full((n * k,), -1, dtype=torch.int32, device="cuda")
        rs = torch.full((n * k,), -1, dtype=torch.int32, device="cuda")
        inv = torch.full((n, k), -1, dtype=torch.int32, device="cuda")
        route = B.spa_route_bufs(idx.data_ptr(), w.data_ptr(), offs.data_ptr(), rt.data_ptr(), rs.data_ptr(),
                                 inv.data_ptr())
        B.spa_moe_route(ctx, m, lay, hn, n, logits, route, None, ws)
        torch.cuda.synchronize()
        assert B.spa_workspace_errors(ctx, ws) == 0
        lg = logits.cpu().numpy().astype(np.float64)
        assert np.isfinite(lg).all() and np.ptp(lg) > 0
        # picks in pick order: the larger logit first, equal logits to the lower index
        expert = np.broadcast_to(np.arange(E), lg.shape)
        want = np.lexsort((expert, -lg), axis=-1)[:, :k]
        got = idx.cpu().numpy()
        np.testing.assert_array_equal(got, want, err_msg=f"{n} tokens: picks")
        # softmax over the picks
        v = np.take_along_axis(lg, want, 1)
        e = np.exp(v - v[:, :1])
        np.testing.assert_allclose(w.cpu().numpy(), e / e.sum(1, keepdims=True), rtol=1e-5, atol=1e-7,
                                   err_msg=f"{n} tokens: weights")
        # the dispatch permutation of these picks, bit for bit
        counts, o_ref, rt_ref, rs_ref, inv_ref = permutation(got.astype(np.int64) % Er, Er)
        np.testing.assert_array_equal(offs.cpu().numpy(), o_ref, err_msg=f"{n} tokens: offsets")
        np.testing.assert_array_equal(rt.cpu().numpy(), rt_ref, err_msg=f"{n} tokens: row tokens")
        np.testing.assert_array_equal(rs.cpu().numpy(), rs_ref, err_msg=f"{n} tokens: row picks")
        np.testing.assert_array_equal(inv.cpu().numpy(), inv_ref, err_msg=f"{n} tokens: inverse")
    B.spa_shutdown(ctx)
