"""Pins of the oracle's W4A8 pieces (int8 activations with a static per-tensor
scale, the FastDeploy page's "W4A8 static quantization"): closed forms of the
activation quantizer (exact grid points, ties to even, clamping), its float32
decision checked against an independent numpy float32 computation, the
reduction to the pinned plain linear layer when the activations lie on the
grid, and the quantization error bound."""
import numpy as np

import oracle
import workloads


def test_grid_points_map_to_their_index():
    s = 0.125                                   # power of two: every product is exact
    k = np.arange(-127, 128, dtype=np.float32)
    assert np.array_equal(oracle.quantize_act(k * np.float32(s), s), k.astype(np.int8))


def test_ties_round_to_even_and_range_clamps():
    s = 0.5
    x = np.array([0.25, 0.75, 1.25, -0.25, -0.75, 63.25, 63.75, 64.0, 1e6, -1e6, -63.75],
                 dtype=np.float32)
    # x / s = 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, 127.5, 128, 2e6, -2e6, -127.5
    assert oracle.quantize_act(x, s).tolist() == [0, 2, 2, 0, -2, 126, 127, 127, 127, -127, -127]
    assert oracle.quantize_act(np.array([np.nan, np.inf, -np.inf], np.float32), s).tolist() == \
        [-127, 127, -127]


def test_float32_decision_matches_numpy_float32():
    g = np.random.default_rng(3)
    x = g.standard_normal(20000).astype(np.float32)
    for s in (0.0123, 3.0 / 127.0, 0.02, 1.7):
        r = np.float32(1.0) / np.float32(s)
        ref = np.clip(np.rint(x * r), -127, 127).astype(np.int8)   # numpy float32 product
        assert np.array_equal(oracle.quantize_act(x, s), ref)


def test_on_grid_activations_reduce_to_the_plain_linear():
    N, K, T = 6, 384, 3
    w = workloads.weights(31, 0, N, K, 0.005, 0.02)
    g = np.random.default_rng(4)
    s = 2.0 ** -5
    x = (g.integers(-127, 128, size=(T, K)) * s).astype(np.float32)
    y, S, a = oracle.linear_w4a8(x, s, w["qweight"], w["scales"], w["zeros"], N, K)
    y0, S0 = oracle.linear(x.astype(np.float64), w["qweight"], w["scales"], w["zeros"], N, K)
    assert np.array_equal(y, y0) and np.array_equal(S, S0)
    assert np.array_equal(a.astype(np.float64) * s, x)


def test_quantization_error_bound():
    # without clamping, |a s - x| <= s / 2 (plus the float32 rounding of x * r), so
    # |y_w4a8 - y| <= (s / 2 + eps) * sum_k |w_k|
    N, K, T = 5, 512, 4
    w = workloads.weights(32, 0, N, K, 0.005, 0.02)
    x = workloads.bf16_bits_to_f32(workloads.activations(32, 1, T, K, "bf16"))
    s = float(np.abs(x).max()) / 127.0
    y, _, a = oracle.linear_w4a8(x, s, w["qweight"], w["scales"], w["zeros"], N, K)
    y0, _ = oracle.linear(x.astype(np.float64), w["qweight"], w["scales"], w["zeros"], N, K)
    wabs = np.abs(oracle.dequant(w["qweight"], w["scales"], w["zeros"], N, K)).sum(axis=1)
    assert np.all(np.abs(a.astype(np.float64) * np.float32(s) - x) <= s * (0.5 + 1e-5))
    assert np.all(np.abs(y - y0) <= (s * (0.5 + 1e-5)) * wabs[None, :])
    assert np.abs(a).max() == 127 and np.abs(y - y0).max() > 0
