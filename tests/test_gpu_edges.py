"""Edge cases of the decode layer on the GPU against the CPU oracle:

* ragged and short KV lengths (1 .. 300: below, at and above the 128-slot
  window, on and off 32-position block boundaries), many resident experts
  (about one row each), an odd batch split into 3 microbatches, spatial equal
  to temporal;
* the first decode step of a single sequence (KV length 1: only the new token
  and the sink), one token through the whole path;
* the largest microbatch the library takes (tokens * top_k = 4096), sampled.
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
