"""Pins of the oracle's rotary position embedding (Figure 3 "RoPE" of the
SubGPU Pipelining paper; the formulation of RoFormer: adjacent pairs of a
head turned by pos * theta^(-2i/D)). Each check rests on something other than
the oracle's own formula: hand-computed values, the complex-number form of a
rotation, the relative-position identity that motivates the method, and the
whole layer at position 0."""
import dataclasses
import math

import numpy as np
import pytest

from oracle import layer as ol


def test_small_head_by_hand():
    # D = 4, theta = 1e4: pair 0 turns by pos, pair 1 by pos / 100
    out = ol.rope(np.array([1.0, 0.0, 1.0, 0.0]), 100, 1e4)
    np.testing.assert_allclose(out, [math.cos(100), math.sin(100), math.cos(1), math.sin(1)], rtol=0, atol=1e-14)
    out = ol.rope(np.array([0.0, 1.0, 0.0, 1.0]), 100, 1e4)
    np.testing.assert_allclose(out, [-math.sin(100), math.cos(100), -math.sin(1), math.cos(1)], rtol=0, atol=1e-14)
    # D = 2: one pair turned by pos radians whatever theta is
    out = ol.rope(np.array([3.0, -2.0]), 7, 123.0)
    c, s = math.cos(7), math.sin(7)
    np.testing.assert_allclose(out, [3 * c + 2 * s, 3 * s - 2 * c], rtol=0, atol=1e-14)


def test_position_zero_is_identity_and_pair_norms_are_kept():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64))
    np.testing.assert_array_equal(ol.rope(x, 0, 10000.0), x)
    y = ol.rope(x, 4321, 10000.0)
    np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-13)


@pytest.mark.parametrize("pos,theta", [(1, 10000.0), (8191, 10000.0), (32767, 150000.0)])
def test_equals_complex_multiplication(pos, theta):
    rng = np.random.default_rng(2)
    D = 64
    x = rng.standard_normal((2, D))
    freqs = 1.0 / theta ** (np.arange(0, D, 2) / D)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos * freqs)
    ref = np.empty_like(x)
    ref[:, 0::2], ref[:, 1::2] = z.real, z.imag
    # the two forms round the angle differently: ~1e-16 relative times pos
    np.testing.assert_allclose(ol.rope(x, pos, theta), ref, rtol=0, atol=1e-15 * pos + 1e-14)


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(10, 3), (500, 499), (4000, 17)]:
        a = ol.rope(q, m, 10000.0) @ ol.rope(k, n, 10000.0)
        b = ol.rope(q, m - n, 10000.0) @ k
        assert abs(a - b) < 1e-10 * (1 + abs(b))


def test_layer_at_position_zero_equals_layer_without_rope():
    """Every sequence decoding its first token (L = 1): the rotation is the
    identity, so the whole layer is unchanged bit for bit."""
    from tests.test_oracle_layer import _history, _params, _tiny, rnd
    dims = _tiny()
    rng = np.random.default_rng(4)
    dense, experts = _params(dims, rng)
    _, _, hist = _history(dims, rng, 3, 4)
    x = rnd(rng, 3, dims.hidden)
    off = ol.layer_forward(dims, ol.Numerics("bf16", "bf16", "bf16"), "full", x, dense, experts.__getitem__,
                           [1, 1, 1], hist)
    on = ol.layer_forward(dataclasses.replace(dims, rope_theta=10000.0), ol.Numerics("bf16", "bf16", "bf16"),
                          "full", x, dense, experts.__getitem__, [1, 1, 1], hist)
    np.testing.assert_array_equal(on.x_next, off.x_next)
    np.testing.assert_array_equal(on.q, off.q)


def test_rope_moves_the_layer_when_positions_are_nonzero():
    from tests.test_oracle_layer import _history, _params, _tiny, rnd
    dims = _tiny()
    rng = np.random.default_rng(5)
    dense, experts = _params(dims, rng)
    _, _, hist = _history(dims, rng, 2, 10)
    x = rnd(rng, 2, dims.hidden)
    off = ol.layer_forward(dims, ol.Numerics(), "full", x, dense, experts.__getitem__, [9, 5], hist)
    on = ol.layer_forward(dataclasses.replace(dims, rope_theta=10000.0), ol.Numerics(), "full", x, dense,
                          experts.__getitem__, [9, 5], hist)
    assert np.max(np.abs(on.q - off.q)) > 1e-3
    np.testing.assert_array_equal(on.v_new, off.v_new)      # values are not rotated
