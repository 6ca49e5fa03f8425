"""Attention shapes the headline workloads do not reach, and the pages' own
KV length, against the CPU oracle (teacher-forced per layer, every sampled
sequence element by element):

* more than 8 chunks per window: two sequences with KV lengths in
  [8192, 16384] leave too few (sequence, KV head) pairs to fill two workgroups
  per CU, so the chunk drops to 512 positions and a full window has 16-32
  chunks; the chunk states are merged by the general (two-pass) merge, and
  the dealt full-layer kernel deals many chunks per sequence;
* 16 query heads per KV head (G * D = 1024 > 512, the general merge again)
  at 264 sequences: the dealt kernel's pieces merged by the general merge;
* 1,040 sequences with top-2 routing, above the dealt kernel's 1,024 tokens:
  the per-chunk grid kernel runs the full layer (windows of 2-3 chunks);
* KV length 32,768 for every sequence (the SubGPU Pipelining paper's section
  5.1 shape): the first sliding and the first full layer of the 36-layer
  share, all 64 sequences, in the tuned launch configuration.
"""
import pytest

from tests import harness as hz
from tests.test_gpu_iteration import teacher_forced, tuned

pytestmark = pytest.mark.gpu


def test_many_chunks_general_merge_dealt_kernel():
    from spatially_pipelined_attention_amd import synth
    wl = synth.WORKLOADS["gptoss_36l_b64"].with_(
        name="wide_chunks", seed=2011, batch=2, kv_len_lo=8192, kv_len_hi=16384, n_layers=1,
        layer_kinds=("full",))
    toks = list(range(wl.batch))
    print(f"\n[wide_chunks] L = {synth.kv_lengths(wl).tolist()}", flush=True)
    resample, _ = hz.resample_for_margins(wl, toks)
    teacher_forced(wl, toks, resample, {"cut": 0, "n_micro": 1, "cu_a": 0})
    teacher_forced(wl, toks, resample, {"cut": 0, "n_micro": 2, "cu_a": 128})


def test_sixteen_heads_per_group_general_merge_dealt_kernel():
    from spatially_pipelined_attention_amd import synth
    import numpy as np
    wl = synth.WORKLOADS["gptoss_36l_b64"].with_(
        name="wide_g16", seed=2012, n_kv_heads=4, batch=264, kv_len_lo=1024, kv_len_hi=6000, n_layers=2,
        layer_kinds=("sliding", "full"))
    L = synth.kv_lengths(wl)
    long_toks = [int(t) for t in np.argsort(-L)[:6]]          # the longest windows: cut into pieces
    toks = sorted(set(long_toks + [0, 131, 263]))
    print(f"\n[wide_g16] sampled L = {[int(L[t]) for t in toks]}", flush=True)
    resample, _ = hz.resample_for_margins(wl, toks)
    teacher_forced(wl, toks, resample, {"cut": 0, "n_micro": 1, "cu_a": 0})


def test_past_the_split_limit_grid_kernel():
    from spatially_pipelined_attention_amd import synth
    import numpy as np
    wl = synth.WORKLOADS["gptoss_36l_b64"].with_(
        name="wide_grid", seed=2013, top_k=2, batch=1040, kv_len_lo=1024, kv_len_hi=3000, n_layers=2,
        layer_kinds=("sliding", "full"))
    L = synth.kv_lengths(wl)
    long_toks = [int(t) for t in np.argsort(-L)[:4]]          # the longest windows: several chunks
    toks = sorted(set(long_toks + [0, 517, 1039]))
    print(f"\n[wide_grid] sampled L = {[int(L[t]) for t in toks]}", flush=True)
    resample, _ = hz.resample_for_margins(wl, toks)
    teacher_forced(wl, toks, resample, {"cut": 0, "n_micro": 1, "cu_a": 0})


def test_paper_shape_kv32k_first_layers_all_sequences():
    from spatially_pipelined_attention_amd import synth
    base = synth.WORKLOADS["gptoss_36l_kv32k"]
    wl = base.with_(n_layers=2, layer_kinds=base.layer_kinds[:2])
    toks = list(range(wl.batch))
    resample, _ = hz.resample_for_margins(wl, toks, n_layers=2)
    teacher_forced(wl, toks, resample, tuned("gptoss_36l_kv32k", wl.batch))
