"""The no-allocation decode attention entry point (spa_decode_attn_noalloc)
against spa_decode_attn with a workspace, through the C ABI, on the GPU.

Both run the same kernels over the same pieces, so the outputs must be
identical bit for bit. Two calls in a row: a full layer over all 64
sequences (the launch's blocks split evenly over the device's ranges), then
a smaller call of 16 sequences (another split), which must not see anything
the first call left in the fixed scratch array; then a sliding layer, and a
full layer of 1,040 sequences with top-2 routing (above the split kernel's
1,024 tokens: one workgroup per chunk). A call whose partials would not fit
the array is refused before any launch.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_noalloc_attention_equals_workspace_attention_twice():
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    wl0 = synth.WORKLOADS["gptoss_36l_b64"]
    wl = wl0.with_(n_layers=2, layer_kinds=wl0.layer_kinds[:2])      # sliding, full
    print("\n[no-alloc] building a 2-layer slice of gptoss_36l_b64", flush=True)
    dw = DeviceWorkload(wl)
    ctx = B.spa_init(0)
    QD = wl.n_q_heads * wl.head_dim
    gen = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn(wl.batch, QD, device="cuda", generator=gen).to(torch.bfloat16)
    for layer, tok0, n_tok in ((1, 0, 64), (1, 40, 16), (0, 3, 9)):
        print(f"[no-alloc] layer {layer} ({wl.layer_kinds[layer]}), tokens {tok0}..{tok0 + n_tok - 1}", flush=True)
        qs = q[tok0:tok0 + n_tok].contiguous()
        ws = dw.workspace(n_tok=n_tok)
        o_ref = torch.empty(n_tok, QD, dtype=torch.bfloat16, device="cuda")
        o_got = torch.full_like(o_ref, float("nan"))
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.spa_decode_attn(ctx, dw.m, dw.layers_c[layer], dw.batch, tok0, n_tok, qs, o_ref, ws)
        B.spa_decode_attn_noalloc(ctx, dw.m, dw.layers_c[layer], dw.batch, tok0, n_tok, qs, o_got, err)
        torch.cuda.synchronize()
        assert torch.equal(o_ref, o_got), f"layer {layer}, tokens {tok0}+{n_tok}"
        assert int(err.item()) == 0 and B.spa_workspace_errors(ctx, ws) == 0
    del dw
    # 1,040 sequences: the per-chunk grid kernel, whose partials grow with
    # the batch's length bound
    wl2 = wl.with_(name="noalloc_grid", seed=2017, top_k=2, batch=1040, kv_len_lo=16, kv_len_hi=200)
    print("[no-alloc] layer 1 (full), 1040 tokens", flush=True)
    dw2 = DeviceWorkload(wl2)
    q2 = torch.randn(wl2.batch, QD, device="cuda", generator=gen).to(torch.bfloat16)
    ws = dw2.workspace(n_tok=wl2.batch)
    o_ref = torch.empty(wl2.batch, QD, dtype=torch.bfloat16, device="cuda")
    o_got = torch.full_like(o_ref, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.spa_decode_attn(ctx, dw2.m, dw2.layers_c[1], dw2.batch, 0, wl2.batch, q2, o_ref, ws)
    B.spa_decode_attn_noalloc(ctx, dw2.m, dw2.layers_c[1], dw2.batch, 0, wl2.batch, q2, o_got, err)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o_got), "full layer, 1040 tokens"
    assert int(err.item()) == 0 and B.spa_workspace_errors(ctx, ws) == 0
    # partials beyond the fixed array: refused on the host, nothing launched
    big = B.spa_batch.from_buffer_copy(dw2.batch)
    big.max_kv_len = 10_000_000
    with pytest.raises(B.SpaError) as ei:
        B.spa_decode_attn_noalloc(ctx, dw2.m, dw2.layers_c[1], big, 0, wl2.batch, q2, o_got)
    assert ei.value.status == B.SPA_EWORKSPACE
    B.spa_shutdown(ctx)
