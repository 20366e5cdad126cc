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


# ---- the W4A8 MoE layer ----------------------------------------------------------

def _small_moe(seed, E=4, H=256, I=128):
    ex = workloads.moe_experts(seed, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(seed, 0, H, I, 0.005, 0.02)
    x = workloads.bf16_bits_to_f32(workloads.activations(seed, 1, 3, H, "bf16"))
    return ex, sh, x, E, H, I


def test_moe_w4a8_top1_is_the_chain_of_pinned_pieces():
    # one expert with weight 1, no shared one: xhat from the activation quantizer,
    # h = SiLU(g) * u (pinned gate_up_silu), h quantized the same way, then the
    # pinned linear layer
    ex, _, x, E, H, I = _small_moe(41)
    sx, shh = float(np.abs(x).max()) / 127.0, 0.05
    ids = np.array([[2], [0], [3]], dtype=np.int32)
    out, tol = oracle.moe_w4a8(x, sx, shh, ids, np.ones((3, 1)), ex, None, H, I, E)
    xh = oracle.dequant_act(oracle.quantize_act(x, sx), sx)
    for t in range(3):
        e = ids[t, 0]
        h, _ = oracle.gate_up_silu(xh[t:t + 1], ex["gu_q"][e], ex["gu_s"][e], ex["gu_z"][e], I, H)
        hh = oracle.dequant_act(oracle.quantize_act(h.astype(np.float32), shh), shh)
        y, S = oracle.linear(hh, ex["dn_q"][e], ex["dn_s"][e], ex["dn_z"][e], H, I)
        assert np.array_equal(out[t], y[0])
        assert np.all(tol[t] >= oracle.C_TOL * S[0] * (1 - 1e-12))


def test_moe_w4a8_fine_h_grid_approaches_the_plain_layer_on_xhat():
    # with a fine h grid the int8 h step vanishes: |out - moe(xhat)| <= s_h / 2 *
    # sum of |W_d| over the selected experts and the shared one (clamping off:
    # s_h * 127 above every |h|)
    ex, sh, x, E, H, I = _small_moe(42)
    sx = float(np.abs(x).max()) / 127.0
    ids = np.array([[1, 3], [0, 2], [3, 0]], dtype=np.int32)
    pw = np.array([[0.75, 0.25], [0.5, 0.5], [0.1, 0.9]])
    xh = oracle.dequant_act(oracle.quantize_act(x, sx), sx)
    ref, _ = oracle.moe(xh, ids, pw, ex, sh, H, I, E)
    hmax = 0.0
    for e in range(E):
        h, _ = oracle.gate_up_silu(xh, ex["gu_q"][e], ex["gu_s"][e], ex["gu_z"][e], I, H)
        hmax = max(hmax, float(np.abs(h).max()))
    hs, _ = oracle.gate_up_silu(xh, sh["gu_q"], sh["gu_s"], sh["gu_z"], I, H)
    hmax = max(hmax, float(np.abs(hs).max()))
    shh = hmax / 127.0
    out, _ = oracle.moe_w4a8(x, sx, shh, ids, pw, ex, sh, H, I, E)
    wd = [np.abs(oracle.dequant(ex["dn_q"][e], ex["dn_s"][e], ex["dn_z"][e], H, I)).sum(axis=1)
          for e in range(E)]
    wsh = np.abs(oracle.dequant(sh["dn_q"], sh["dn_s"], sh["dn_z"], H, I)).sum(axis=1)
    for t in range(3):
        bound = shh * (0.5 + 1e-5) * (sum(pw[t, j] * wd[ids[t, j]] for j in range(2)) + wsh)
        assert np.all(np.abs(out[t] - ref[t]) <= bound)
    assert np.abs(out - ref).max() > 0


def test_moe_w4a8_zero_weights_leave_the_shared_expert():
    ex, sh, x, E, H, I = _small_moe(43)
    sx, shh = float(np.abs(x).max()) / 127.0, 0.02
    ids = np.array([[0, 1], [2, 3], [1, 2]], dtype=np.int32)
    out, _ = oracle.moe_w4a8(x, sx, shh, ids, np.zeros((3, 2)), ex, sh, H, I, E)
    only, _ = oracle.moe_w4a8(x, sx, shh, ids[:, :1], np.zeros((3, 1)), ex, sh, H, I, E)
    assert np.array_equal(out, only) and np.abs(out).max() > 0
