"""Why long chains are compared schedule against schedule, not against the
oracle (CPU, the oracle alone).

The 36-layer workload's residual stream is sensitive to bf16-sized changes:
after a relative change of 2^-9 (one bf16 rounding step) to one element of
one sequence's input, the oracle's own outputs drift past the 2e-2 x RMS bar
within eleven layers, before any expert pick changes, and at layer 14 a pick
flips. (Over all 36 layers the same change moves the output by 4-48% of RMS
for the sequences tried.) A GPU chain whose mirrored rounding points straddle a
rounding boundary somewhere (both sides sum in another order) sees changes of
that size, so over many layers it cannot be held to the oracle element by
element; per-layer teacher-forced checks and the spatial = temporal identity
cover the chain instead.
"""
import numpy as np
import pytest

from oracle import layer as ol
from spatially_pipelined_attention_amd import synth
from tests import harness as hz

pytestmark = pytest.mark.slow


def test_one_bf16_step_in_one_input_element_flips_a_pick_downstream():
    name, tok, elem, n_layers, flip_layer = "gptoss_36l_b64", 3, 0, 15, 14
    wl = synth.WORKLOADS[name]
    x0 = synth.x_rows(wl, [tok], hz.load_resample(name)).astype(np.float64)[0]
    x1 = x0.copy()
    x1[elem] *= 1.0 + 2.0 ** -9
    L = [int(synth.kv_lengths(wl)[tok])] * 2
    x = np.stack([x0, x1])
    picks, drift = [], []
    for l in range(n_layers):
        dense, expert = hz.layer_params(wl, l)
        rec = ol.layer_forward(hz.dims(wl), hz.numerics(wl), wl.layer_kinds[l], x, dense, expert, L,
                               lambda b, lo, hi, _l=l: synth.kv_history(wl, _l, tok, lo, hi))
        x = rec.x_next
        picks.append(np.sort(rec.topk, axis=1))
        rms = float(np.sqrt(np.mean(x[0] ** 2)))
        print(f"layer {l}: picks equal {np.array_equal(picks[-1][0], picks[-1][1])}, "
              f"max|diff|/RMS {np.max(np.abs(x[1] - x[0])) / rms:.2e}, margin {rec.margin[0]:.2e}")
        drift.append(np.max(np.abs(x[1] - x[0])) / rms)
    same = [np.array_equal(p[0], p[1]) for p in picks]
    assert all(same[:flip_layer]), "the picks agree up to the flip"
    assert not same[flip_layer], "a pick flips at layer 14"
    assert drift[0] < hz.TOL["bf16"] < max(drift[:flip_layer]), "the drift passes the bar before any flip"
