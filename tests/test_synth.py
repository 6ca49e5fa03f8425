"""The seeded generator: determinism, slice independence and moments (CPU)."""
import numpy as np
import pytest


def test_same_seed_same_bits_and_slices_regenerate(synth):
    k = synth.stream_key(7, synth.TAG_KHIST, 3, 0)
    a = synth.normal_bf16_bits(10000, k, 0, 1.0)
    b = synth.normal_bf16_bits(10000, k, 0, 1.0)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(synth.normal_bf16_bits(100, k, 5000, 1.0), a[5000:5100])
    assert not np.array_equal(a, synth.normal_bf16_bits(10000, synth.stream_key(7, synth.TAG_KHIST, 4, 0), 0, 1.0))


def test_bf16_stream_is_rounded_f32_stream(synth):
    import torch
    k = synth.stream_key(11, synth.TAG_WQKV)
    f = synth.normal_f32(50000, k, 0, 0.02)
    bits = synth.normal_bf16_bits(50000, k, 0, 0.02)
    ref = torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_normal_moments(synth):
    a = synth.normal_f32(2_000_000, synth.stream_key(3, 1), 0, 1.0).astype(np.float64)
    assert abs(a.mean()) < 3e-3
    assert abs(a.std() - 1.0) < 3e-3
    assert abs(a.max()) <= 2 * np.sqrt(3) + 1e-6
    # Irwin-Hall(4) kurtosis: 3 - 6/(5*4) = 2.7
    assert abs(((a - a.mean()) ** 4).mean() / a.var() ** 2 - 2.7) < 0.02


def test_kv_lengths_in_range(synth):
    wl = synth.WORKLOADS["gptoss_36l_b64"]
    L = synth.kv_lengths(wl)
    assert L.shape == (64,) and L.min() >= 1024 and L.max() <= 8192
    assert len(set(L.tolist())) > 50


def test_kv_history_slices_agree(synth):
    wl = synth.WORKLOADS["gptoss_36l_b64"]
    K, V = synth.kv_history(wl, 1, 5, 100, 160)
    K2, V2 = synth.kv_history(wl, 1, 5, 130, 140)
    np.testing.assert_array_equal(K[:, 30:40], K2)
    np.testing.assert_array_equal(V[:, 30:40], V2)
    assert not np.array_equal(K, V)


def test_x_resample_changes_only_that_token(synth):
    wl = synth.WORKLOADS["gptoss_layer_full"]
    a = synth.x_rows(wl, [0, 1, 2])
    b = synth.x_rows(wl, [0, 1, 2], {1: 3})
    np.testing.assert_array_equal(a[[0, 2]], b[[0, 2]])
    assert not np.array_equal(a[1], b[1])
