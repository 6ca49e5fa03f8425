"""Edge cases of the decode layer on the GPU against the CPU oracle:

* ragged and short KV lengths (1 .. 300: below, at and above the 128-slot
  window, on and off 32-position block boundaries), many resident experts
  (about one row each), an odd batch split into 3 microbatches, spatial equal
  to temporal;
* 256 router experts with top-8 picks, temporal and spatial;
* the first decode step of a single sequence (KV length 1: only the new token
  and the sink), one token through the whole path;
* the largest microbatch the library takes (tokens * top_k = 4096), sampled;
* 256 tokens in bf16 and fp8 (the LDS-tiled products of 128-row blocks), sampled.
Inputs come from the seeded generator with new seeds; router re-draws for the
margin are computed here by the oracle.
"""
import numpy as np
import pytest
import torch

from tests import harness as hz

pytestmark = pytest.mark.gpu


def _setup(wl, toks):
    from spatially_pipelined_attention_amd import binding as B
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    resample, _ = hz.resample_for_margins(wl, toks)
    x_ref, picks, margins, _ = hz.run_oracle(wl, toks, resample)
    dw = DeviceWorkload(wl, resample)
    ctx = B.spa_init(0)
    return B, dw, ctx, x_ref, picks


def _run(B, ctx, dw, cfg):
    from spatially_pipelined_attention_amd.workload import Pipeline
    pipe = Pipeline(ctx, dw.m, cfg)
    ws = dw.workspace(n_micro=cfg["n_micro"])
    dw.reset_x()
    dw.topk.zero_()
    pipe.run(dw.layers_c, dw.batch, ws)
    torch.cuda.synchronize()
    pipe.close()
    assert B.spa_workspace_errors(ctx, ws) == 0
    return dw.x.clone(), dw.topk.clone()


def _same_picks(got, ref):
    return np.array_equal(np.sort(got, axis=-1), np.sort(ref, axis=-1))


def test_ragged_short_lengths_many_experts_odd_batch():
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS["gptoss_layer_full"].with_(
        name="edge_ragged", seed=2001, batch=9, kv_len_lo=1, kv_len_hi=300, n_layers=2,
        layer_kinds=("sliding", "full"))
    toks = list(range(wl.batch))
    print(f"\n[edge_ragged] L = {synth.kv_lengths(wl).tolist()}", flush=True)
    B, dw, ctx, x_ref, picks = _setup(wl, toks)
    x1, t1 = _run(B, ctx, dw, {"cut": 0, "n_micro": 1, "cu_a": 0})
    hz.assert_close_rms(x1.double().cpu().numpy(), x_ref, hz.tol_of(wl), "T1 vs oracle")
    assert _same_picks(t1.cpu().numpy(), picks)
    xt, tt = _run(B, ctx, dw, {"cut": 1, "n_micro": 3, "cu_a": 0})
    xs, ts = _run(B, ctx, dw, {"cut": 1, "n_micro": 3, "cu_a": 96})
    assert torch.equal(xt, xs) and torch.equal(tt, ts)
    hz.assert_close_rms(xs.double().cpu().numpy(), x_ref, hz.tol_of(wl), "T3 spatial vs oracle")


def test_wide_router_and_eight_picks():
    """256 router experts (each lane of the top-k wave holds four logits) and
    top-8 (the combine's general pick loop; at most 4 picks take its batched
    form), temporal and spatial."""
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS["gptoss_layer_full"].with_(
        name="edge_wide", seed=2007, batch=6, n_experts=256, top_k=8, n_resident=16, kv_len_lo=40,
        kv_len_hi=400, n_layers=2, layer_kinds=("sliding", "full"))
    toks = list(range(wl.batch))
    print("\n[edge_wide] E 256, top-8, 16 resident experts", flush=True)
    B, dw, ctx, x_ref, picks = _setup(wl, toks)
    x1, t1 = _run(B, ctx, dw, {"cut": 0, "n_micro": 1, "cu_a": 0})
    hz.assert_close_rms(x1.double().cpu().numpy(), x_ref, hz.tol_of(wl), "E 256, top-8")
    assert _same_picks(t1.cpu().numpy(), picks)
    xt, tt = _run(B, ctx, dw, {"cut": 0, "n_micro": 2, "cu_a": 0})
    xs, ts = _run(B, ctx, dw, {"cut": 0, "n_micro": 2, "cu_a": 128})
    assert torch.equal(xt, xs) and torch.equal(tt, ts)


def test_first_step_of_a_single_sequence():
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS["gptoss_36l_b64"].with_(
        name="edge_first", seed=2002, batch=1, kv_len_lo=1, kv_len_hi=1, n_layers=2,
        layer_kinds=("sliding", "full"))
    B, dw, ctx, x_ref, picks = _setup(wl, [0])
    x1, t1 = _run(B, ctx, dw, {"cut": 0, "n_micro": 1, "cu_a": 0})
    hz.assert_close_rms(x1.double().cpu().numpy(), x_ref, hz.tol_of(wl), "one token, L = 1")
    assert _same_picks(t1.cpu().numpy(), picks)


def test_largest_microbatch_sampled():
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS["gptoss_36l_b64"].with_(
        name="edge_large", seed=2003, batch=1024, kv_len_lo=64, kv_len_hi=200, n_layers=1,
        layer_kinds=("sliding",))
    toks = [0, 511, 1023]
    B, dw, ctx, x_ref, picks = _setup(wl, toks)
    x1, t1 = _run(B, ctx, dw, {"cut": 0, "n_micro": 1, "cu_a": 0})
    hz.assert_close_rms(x1.double().cpu().numpy()[toks], x_ref, hz.tol_of(wl), "1024 tokens")
    assert _same_picks(t1.cpu().numpy()[:, toks], picks)


@pytest.mark.parametrize("name,n_layers", [("gptoss_36l_fp8", 1), ("gptoss_36l_b64", 2)])
def test_large_batch_expert_tiles_sampled(name, n_layers):
    """256 tokens (about 256 rows per expert, 128-row blocks): the expert and
    dense products take the LDS-tiled kernel, E4M3 scales included for fp8.
    fp8 is held to its bar one layer at a time, as in the iteration tests
    (two chained fp8 layers drift to about 7% of RMS in the oracle
    comparison whichever product kernel runs)."""
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS[name].with_(name=f"edge_big_{name}", seed=2006, batch=256, kv_len_lo=64, kv_len_hi=600,
                                     n_layers=n_layers, layer_kinds=("sliding", "full")[:n_layers])
    toks = [0, 77, 191, 255]
    print(f"\n[case] {name}, 256 tokens, sampled {toks}", flush=True)
    B, dw, ctx, x_ref, picks = _setup(wl, toks)
    x1, t1 = _run(B, ctx, dw, {"cut": 0, "n_micro": 1, "cu_a": 0})
    hz.assert_close_rms(x1.double().cpu().numpy()[toks], x_ref, hz.tol_of(wl), f"256 tokens, {n_layers} layer(s)")
    assert _same_picks(t1.cpu().numpy()[:, toks], picks)


@pytest.mark.parametrize("batch,refused", [(16, (3, 9)), (300, (3, 9, 257, 299))])
def test_kv_length_beyond_capacity_is_refused(batch, refused):
    """A cached length above the sequence's capacity (or zero) sets the
    error bit and is skipped before any KV read; every other token's
    attention output is unchanged (bit for bit on the sliding layer, within
    rounding on the full layer, whose split follows the launch's lengths).
    Each call clears the error word first, so each reading belongs to one
    launch. 16 tokens run the split's one-token-per-thread prologue, 300
    tokens its four-token one."""
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    base = synth.WORKLOADS["gptoss_36l_b64"]
    wl = base.with_(name="edge_refuse", seed=2005, n_layers=2, layer_kinds=("sliding", "full"), batch=batch,
                    kv_len_lo=200, kv_len_hi=600)
    print(f"\n[case] kv length beyond capacity, {batch} tokens, refused {refused}", flush=True)
    dw = DeviceWorkload(wl)
    ctx = B.spa_init(0)
    n = wl.batch
    g = torch.Generator(device="cpu").manual_seed(7)
    q = (torch.randn(n, wl.n_q_heads * wl.head_dim, generator=g) * 0.5).to(torch.bfloat16).to("cuda")
    ws = dw.workspace(n_micro=1)
    outs, errs = [], []
    for bad in (False, True):
        saved = dw.kv_len_d.clone()
        if bad:
            for i, t in enumerate(refused):   # above capacity, or zero
                dw.kv_len_d[t] = dw.kv_cap_d[t] + 1 if i % 2 == 0 else 0
        for layer in (1, 0):   # full (packed cache), then sliding (ring)
            o = torch.zeros_like(q)
            B.spa_decode_attn(ctx, dw.m, dw.layers_c[layer], dw.batch, 0, n, q, o, ws)
            torch.cuda.synchronize()
            outs.append(o.clone())
            errs.append(B.spa_workspace_errors(ctx, ws))
        dw.kv_len_d.copy_(saved)
    assert errs[0] == 0 and errs[1] == 0
    assert errs[2] & 1 and errs[3] & 1
    keep = [t for t in range(n) if t not in refused]
    # full layer: the launch's blocks are split evenly, so a refused token's
    # missing blocks move the other windows' split points. The probabilities
    # enter the PV product in bf16, each relative to its piece's running
    # maximum, so moving a split changes their rounding (2^-9 of each term)
    # and the output's by about 2^-9 of the output scale; the output itself
    # is rounded to bf16 (spacing <= 2^-7 of its magnitude). Bound: 2^-7 of
    # (|element| + RMS of the outputs)
    got = outs[2][keep].double().cpu().numpy()
    ref = outs[0][keep].double().cpu().numpy()
    bound = 2.0 ** -7 * (np.abs(ref) + np.sqrt(np.mean(ref * ref)))
    worst = float((np.abs(got - ref) / bound).max())
    assert worst <= 1.0, f"full layer, refused tokens left out: {worst:.2f} of the rounding bound"
    assert torch.equal(outs[1][keep], outs[3][keep])   # sliding layer: one workgroup per window, bit for bit
