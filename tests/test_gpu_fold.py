"""The QKV finish folded into the sliding-layer attention, against the separate
finish kernel on the GPU, bit for bit.

One sliding layer of the 36-layer workload (64 sequences: the attention runs
one wave per window, so the layer path folds the finish into that kernel) is
run twice from the same KV cache, at the model's hidden size 2880 (the QKV
product takes 3 splits: the finish's bound is 4, one +0 term), at 512 and 256
(2 splits and 1: no padding term), at 16 sequences (half a window per CU
of a 256-CU device, the smallest launch that takes the kernel there), and with
ragged KV lengths from 1 to 300 (new slots inside rings not yet full):
through the separate entry points (spa_rms_norm, spa_qkv_append with its
finish kernel, spa_decode_attn with q given, spa_out_proj, spa_moe_route,
spa_moe_expert, spa_moe_combine) and through spa_layer_forward. The folded
kernel sums q and the new K/V with the finish kernel's split-sum rule and
rounding, and attends the values the finish would have stored, so the
appended K/V rows of every sequence and the layer output must be equal
exactly, not just within the oracle's tolerance.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hidden,batch,kv", [(2880, 64, None), (512, 64, None), (256, 64, None), (2880, 16, None),
                                             (2880, 64, (1, 300))])
def test_folded_finish_matches_the_separate_kernels(hidden, batch, kv):
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    wl = synth.WORKLOADS["gptoss_36l_b64"]
    wl = wl.with_(n_layers=1, layer_kinds=("sliding",), hidden=hidden, inter=hidden, batch=batch)
    if kv:   # ragged lengths from 1: rings not yet full, and single-position windows
        wl = wl.with_(kv_len_lo=kv[0], kv_len_hi=kv[1])
    print(f"\n[fold] one sliding layer of gptoss_36l_b64, hidden {hidden}, batch {batch}, KV {kv}", flush=True)
    dw = DeviceWorkload(wl)
    ctx = B.spa_init(0)
    m, lay, t0, dev = dw.m, dw.layers_c[0], dw.layers_t[0], dw.dev
    n, H, QD, k = wl.batch, wl.hidden, wl.n_q_heads * wl.head_dim, wl.top_k
    k0, v0 = t0["k_cache"].clone(), t0["v_cache"].clone()
    seqs = list(range(n))
    pos = [int(dw.L[b]) - 1 for b in seqs]
    ws = dw.workspace(n_tok=n)

    print("[fold] separate kernels", flush=True)
    dw.reset_x()
    xn = torch.zeros((n, H), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((n, QD), dtype=torch.bfloat16, device=dev)
    o = torch.zeros((n, QD), dtype=torch.bfloat16, device=dev)
    h = torch.zeros((n, H), dtype=torch.float32, device=dev)
    hn = torch.zeros((n, H), dtype=torch.float32, device=dev)
    logits = torch.zeros((n, wl.n_experts), dtype=torch.float32, device=dev)
    idx = torch.zeros((n, k), dtype=torch.int32, device=dev)
    w = torch.zeros((n, k), dtype=torch.float32, device=dev)
    offs = torch.zeros(wl.n_resident + 1, dtype=torch.int32, device=dev)
    rt = torch.zeros(n * k, dtype=torch.int32, device=dev)
    rs = torch.zeros(n * k, dtype=torch.int32, device=dev)
    inv = torch.zeros((n, k), dtype=torch.int32, device=dev)
    y = torch.zeros((n * k, H), dtype=torch.float32, device=dev)
    xo = torch.zeros((n, H), dtype=torch.float32, device=dev)
    route = B.spa_route_bufs(idx.data_ptr(), w.data_ptr(), offs.data_ptr(), rt.data_ptr(), rs.data_ptr(),
                             inv.data_ptr())
    B.spa_rms_norm(ctx, m, dw.x, t0["gamma1"], n, xn)
    B.spa_qkv_append(ctx, m, lay, dw.batch, 0, n, xn, q, ws)
    B.spa_decode_attn(ctx, m, lay, dw.batch, 0, n, q, o, ws)
    B.spa_out_proj(ctx, m, lay, dw.x, o, n, h, hn, ws)
    B.spa_moe_route(ctx, m, lay, hn, n, logits, route, None, ws)
    B.spa_moe_expert(ctx, m, lay, hn, n, route, y, ws)
    B.spa_moe_combine(ctx, m, h, y, route, n, xo)
    torch.cuda.synchronize()
    assert B.spa_workspace_errors(ctx, ws) == 0
    k_sep, v_sep = dw.read_kv(0, seqs, pos)

    print("[fold] layer path, the finish folded into the attention", flush=True)
    t0["k_cache"].copy_(k0)
    t0["v_cache"].copy_(v0)
    dw.reset_x()
    ws2 = dw.workspace(n_tok=n)
    B.spa_layer_forward(ctx, m, lay, 0, dw.batch, 0, n, ws2)
    torch.cuda.synchronize()
    assert B.spa_workspace_errors(ctx, ws2) == 0
    k_fold, v_fold = dw.read_kv(0, seqs, pos)

    np.testing.assert_array_equal(k_fold, k_sep, err_msg="appended K rows")
    np.testing.assert_array_equal(v_fold, v_sep, err_msg="appended V rows")
    assert np.abs(k_fold).max() > 0 and np.abs(v_fold).max() > 0   # the rows hold data
    diff = (dw.x - xo).abs()
    assert torch.equal(dw.x, xo), f"layer output differs: {int((diff > 0).sum())} elements, max {float(diff.max())}"
    B.spa_shutdown(ctx)
