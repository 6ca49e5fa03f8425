"""The rotary position embedding (Figure 3 "RoPE") on the GPU against the CPU
oracle: q and the new k of every token turned at its decoded position, the
whole two-layer iteration with it, the spatial pipeline equal to the temporal
schedule with the same microbatches, and position 0 (a sequence's first
token) leaving every bit unchanged. Runs a two-layer (sliding, full) slice of
the 36-layer one-GPU workload with rotation base 10000."""
import numpy as np
import pytest
import torch

from tests import harness as hz

pytestmark = pytest.mark.gpu

TOKS = [0, 9, 33, 63]


def _f(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def env():
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    wl = synth.WORKLOADS["gptoss_36l_b64_rope"]
    wl = wl.with_(n_layers=2, layer_kinds=wl.layer_kinds[:2])
    print("\n[setup] 2-layer slice of gptoss_36l_b64_rope", flush=True)
    resample, _ = hz.resample_for_margins(wl, TOKS)
    x_ref, picks, _, recs = hz.run_oracle(wl, TOKS, resample, keep_records=True)
    dw = DeviceWorkload(wl, resample)
    ctx = B.spa_init(0)
    return dict(B=B, wl=wl, dw=dw, ctx=ctx, x_ref=x_ref, picks=picks, recs=recs)


def _run(env, cut, n_micro, cu_a):
    from spatially_pipelined_attention_amd.workload import Pipeline
    B, dw, ctx = env["B"], env["dw"], env["ctx"]
    pipe = Pipeline(ctx, dw.m, {"cut": cut, "n_micro": n_micro, "cu_a": cu_a})
    ws = dw.workspace(n_micro=n_micro)
    dw.reset_x()
    dw.topk.zero_()
    pipe.run(dw.layers_c, dw.batch, ws)
    torch.cuda.synchronize()
    pipe.close()
    assert B.spa_workspace_errors(ctx, ws) == 0
    return dw.x.clone(), dw.topk.clone()


def test_q_and_new_k_are_rotated(env):
    B, wl, dw, ctx = env["B"], env["wl"], env["dw"], env["ctx"]
    rec = env["recs"][0]
    n = wl.batch
    tol = hz.tol_of(wl)
    xn = torch.zeros((n, wl.hidden), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((n, wl.n_q_heads * wl.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = dw.workspace(n_tok=n)
    dw.reset_x()
    print("[case] norm + qkv + rope, layer 0", flush=True)
    B.spa_rms_norm(ctx, dw.m, dw.x, dw.layers_t[0]["gamma1"], n, xn)
    B.spa_qkv_append(ctx, dw.m, dw.layers_c[0], dw.batch, 0, n, xn, q, ws)
    torch.cuda.synchronize()
    qg = _f(q).reshape(n, wl.n_q_heads, wl.head_dim)[TOKS]
    hz.assert_close_rms(qg, rec.q, tol, "rotated q")
    L = dw.L
    kk, vv = dw.read_kv(0, TOKS, [int(L[b]) - 1 for b in TOKS])
    hz.assert_close_rms(kk, rec.k_new, tol, "rotated new k")
    hz.assert_close_rms(vv, rec.v_new, tol, "new v (not rotated)")
    assert B.spa_workspace_errors(ctx, ws) == 0


def test_iteration_matches_oracle_and_spatial_equals_temporal(env):
    print("[case] T1, T2 and the spatial pipeline with rope", flush=True)
    x1, t1 = _run(env, 0, 1, 0)
    hz.assert_close_rms(_f(x1)[TOKS], env["x_ref"], hz.tol_of(env["wl"]), "two layers with rope")
    got = t1.cpu().numpy()[:, TOKS]
    assert np.array_equal(np.sort(got, axis=-1), np.sort(env["picks"], axis=-1))
    x2, t2 = _run(env, 1, 2, 0)
    xs, ts = _run(env, 1, 2, 128)
    assert torch.equal(x2, xs) and torch.equal(t2, ts)


def test_first_token_is_unrotated_bit_for_bit():
    """L = 1: the decoded position is 0, the rotation the identity."""
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload, Pipeline
    wl = synth.WORKLOADS["gptoss_36l_b64_rope"].with_(n_layers=2, layer_kinds=("sliding", "full"), batch=8,
                                                     kv_len_lo=1, kv_len_hi=1)
    print("[case] first token, rope on and off", flush=True)
    ctx = B.spa_init(0)
    outs = []
    for theta in (wl.rope_theta, 0.0):
        dw = DeviceWorkload(wl.with_(rope_theta=theta))
        pipe = Pipeline(ctx, dw.m, {"cut": 0, "n_micro": 1, "cu_a": 0})
        ws = dw.workspace(n_micro=1)
        dw.reset_x()
        pipe.run(dw.layers_c, dw.batch, ws)
        torch.cuda.synchronize()
        pipe.close()
        outs.append(dw.x.clone())
        del dw
    assert torch.equal(outs[0], outs[1])
