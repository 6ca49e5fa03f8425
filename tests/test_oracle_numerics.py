"""Pins of the oracle's format helpers against library conversions (CPU)."""
import numpy as np
import pytest
import torch

from oracle import numerics


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))).astype(np.float32)
    # include exact ties: bf16 value + half an ulp
    base = torch.tensor(a[:1000]).to(torch.bfloat16).double().numpy()
    half_ulp = np.sign(base) * np.exp2(np.floor(np.log2(np.abs(base))) - 8)
    ties = (base + half_ulp).astype(np.float32)     # exact: 9 significant bits
    assert np.all(ties.astype(np.float64) == base + half_ulp)
    a = np.concatenate([a, ties])
    ref = torch.tensor(a).to(torch.bfloat16).double().numpy()
    got = numerics.round_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_exact_halfway_goes_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even neighbour is 1
    assert numerics.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert numerics.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert numerics.round_bf16(np.array([-(1.0 + 2.0 ** -8)]))[0] == -1.0


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = numerics.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])
    assert np.nanmax(got) == 448.0 and numerics.e4m3_decode(np.array([1], np.uint8))[0] == 2.0 ** -9


def test_round_e4m3_matches_torch():
    rng = np.random.default_rng(1)
    a = rng.uniform(-448, 448, 100000) * np.exp2(rng.integers(-12, 1, 100000))
    a = a.astype(np.float32).astype(np.float64)
    ref = torch.tensor(a, dtype=torch.float32).to(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(numerics.round_e4m3(a), ref)


def test_round_e4m3_every_value_round_trips():
    vals = numerics.e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = vals[~np.isnan(vals)]
    np.testing.assert_array_equal(numerics.round_e4m3(vals), vals)


def test_pow2_scale_boundaries():
    s = numerics.pow2_scale(np.array([448.0, 448.0001, 224.0, 1.0, 0.0, 896.0, 895.9]))
    np.testing.assert_array_equal(s, [1.0, 2.0, 0.5, 2.0 ** -8, 1.0, 2.0, 2.0])
    v, sc = numerics.quant_rows_pow2_e4m3(np.array([[3.0, -1000.0, 0.5]]))
    assert sc[0] == 4.0                    # 1000/448 = 2.23 -> 4
    np.testing.assert_array_equal(v, numerics.round_e4m3(np.array([[3.0, -1000.0, 0.5]]) / 4.0) * 4.0)


def test_generator_e4m3_quantiser_matches_torch(synth):
    rng = np.random.default_rng(2)
    w = rng.standard_normal((16, 300)).astype(np.float32) * 0.02
    codes, scales = synth.quant_rows_e4m3(w)
    np.testing.assert_allclose(scales, np.abs(w).max(axis=1) / 448.0, rtol=1e-7)
    ref = torch.tensor(w / scales[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
