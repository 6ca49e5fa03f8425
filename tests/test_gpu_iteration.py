"""Full-size decode iterations against the CPU oracle, in the benchmark's own
launch configuration (the tuned spatial pipeline: cut, microbatches, CU pools).

Sequences are independent, so the oracle on a sample of them is exact.

* every layer, teacher-forced: the oracle's input of layer l is fed to the
  pipeline running layer l alone; the output must meet the bar and pick the
  same experts. This is the per-layer bar at every depth.
* chained: a bf16 residual stream drifts by a few bf16 ulps per layer (the
  mirrored rounding points flip where the two sides' sums straddle a rounding
  boundary), so a chain is compared with the oracle on its first four layers
  only; the whole 36-layer chain is checked by the property that the spatial
  and temporal schedules give identical bits.
"""
import ctypes as C
import json
import os

import numpy as np
import pytest
import torch

from tests import harness as hz

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def tuned(name, batch):
    p = os.path.join(ROOT, "spatially_pipelined_attention_amd", "tuned.json")
    cfg = {"cut": 0, "n_micro": 2, "cu_a": 128}
    if os.path.exists(p):
        cfg.update(json.load(open(p)).get(name, {}))
    if batch % cfg["n_micro"]:
        cfg["n_micro"] = 1
    return cfg


class Pipe:
    def __init__(self, B, ctx, m, cfg, spatial=True):
        from spatially_pipelined_attention_amd.workload import Pipeline
        c = dict(cfg)
        if not spatial:
            c["cu_a"] = 0
        self.p = Pipeline(ctx, m, c)
        self.h = self.p.h

    def run(self, layers, batch, ws):
        self.p.run(layers, batch, ws)
        torch.cuda.synchronize()

    def close(self):
        self.p.close()


def same_picks(got, ref):
    """Selection is what must be exact; the order of near-equal picks is not fixed."""
    return np.array_equal(np.sort(got, axis=-1), np.sort(ref, axis=-1))


def teacher_forced(wl, toks, resample, cfg, n_layers=None):
    """Run each layer l alone through the pipeline `cfg`, its input rows set to
    the oracle's input of layer l, and compare every sampled row and its
    expert picks with the oracle's layer output. Returns the worst
    max|err|/RMS."""
    from spatially_pipelined_attention_amd import binding as B
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    name = wl.name
    nl = n_layers or wl.n_layers
    print(f"\n[{name}] oracle on {len(toks)} sequences, {nl} layers", flush=True)
    _, picks, margins, recs = hz.run_oracle(wl, toks, resample, n_layers=nl, keep_records=True)
    assert margins.min() >= hz.MARGIN_MIN, "sampled sequences must clear the router margin"
    x0 = hz.synth.x_rows(wl, toks, resample)
    dw = DeviceWorkload(wl, resample)
    ctx = B.spa_init(0)
    m1 = B.spa_model_desc.from_buffer_copy(dw.m)
    m1.n_layers = 1
    print(f"[{name}] pipeline {cfg}", flush=True)
    pipe = Pipe(B, ctx, m1, cfg)
    topk1 = torch.zeros((1, wl.batch, wl.top_k), dtype=torch.int32, device=dw.dev)
    batch1 = B.spa_batch(wl.batch, dw.max_kv_len, dw.kv_len_d.data_ptr(), dw.kv_off_d.data_ptr(),
                         dw.kv_cap_d.data_ptr(), dw.x.data_ptr(), topk1.data_ptr())
    ws = dw.workspace(n_micro=cfg["n_micro"])
    tol = hz.tol_of(wl)
    worst = 0.0
    try:
        for l in range(nl):
            x_in = x0 if l == 0 else recs[l - 1].x_next
            dw.reset_x()
            dw.x[toks] = torch.as_tensor(x_in, dtype=torch.float32, device=dw.dev)
            pipe.run((B.spa_layer * 1)(dw.layers_c[l]), batch1, ws)
            got = dw.x.double().cpu().numpy()[toks]
            err = hz.assert_close_rms(got, recs[l].x_next, tol, f"{name} layer {l}")
            print(f"  layer {l}: max|err|/RMS {err:.3e}", flush=True)
            worst = max(worst, err)
            assert same_picks(topk1[0].cpu().numpy()[toks], recs[l].topk), f"{name} layer {l}: expert picks"
        assert B.spa_workspace_errors(ctx, ws) == 0
    finally:
        pipe.close()
    print(f"[{name}] worst max|err|/RMS over {nl} layers: {worst:.3e}", flush=True)
    return worst


CASES = ["gptoss_36l_b64", "gptoss_layer_sliding_b256", "gptoss_36l_fp8"]


@pytest.mark.parametrize("name", CASES)
def test_every_layer_teacher_forced(name):
    """Every layer, every sequence of the batch (the dealt attention kernel
    spreads each sequence's chunks over the pool, so every token is checked)."""
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS[name]
    resample = hz.load_resample(name)
    if name == "gptoss_36l_fp8" and not resample:
        pytest.skip("no stored router re-draw map for the fp8 workload")
    teacher_forced(wl, list(range(wl.batch)), resample, tuned(name, wl.batch))


def test_chain_first_layers_matches_oracle():
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    name, toks, nl = "gptoss_36l_b64", [3, 40, 7, 21], 4
    wl0 = synth.WORKLOADS[name]
    wl = wl0.with_(n_layers=nl, layer_kinds=wl0.layer_kinds[:nl])
    resample = hz.load_resample(name)
    x_ref, picks, _, _ = hz.run_oracle(wl, toks, resample)
    dw = DeviceWorkload(wl, resample)
    ctx = B.spa_init(0)
    cfg = tuned(name, wl.batch)
    pipe = Pipe(B, ctx, dw.m, cfg)
    ws = dw.workspace(n_micro=cfg["n_micro"])
    try:
        dw.reset_x()
        pipe.run(dw.layers_c, dw.batch, ws)
    finally:
        pipe.close()
    hz.assert_close_rms(dw.x.double().cpu().numpy()[toks], x_ref, hz.tol_of(wl), "4-layer chain")
    assert same_picks(dw.topk.cpu().numpy()[:, toks], picks)


def test_full_chain_spatial_equals_temporal():
    from spatially_pipelined_attention_amd import binding as B, synth
    from spatially_pipelined_attention_amd.workload import DeviceWorkload
    name = "gptoss_36l_b64"
    wl = synth.WORKLOADS[name]
    dw = DeviceWorkload(wl, hz.load_resample(name))
    ctx = B.spa_init(0)
    cfg = tuned(name, wl.batch)
    out = []
    for spatial in (True, False):
        pipe = Pipe(B, ctx, dw.m, cfg, spatial)
        ws = dw.workspace(n_micro=cfg["n_micro"])
        try:
            dw.reset_x()
            dw.topk.zero_()
            pipe.run(dw.layers_c, dw.batch, ws)
            assert B.spa_workspace_errors(ctx, ws) == 0
        finally:
            pipe.close()
        out.append((dw.x.clone(), dw.topk.clone()))
    assert torch.equal(out[0][0], out[1][0])
    assert torch.equal(out[0][1], out[1][1])
