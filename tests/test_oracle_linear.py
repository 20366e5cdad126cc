"""Pins of the oracle's linear layer and fused SiLU(gate)*up: exact rational brute
force, closed forms, one-hot probes that expose transposed or shifted operands,
linearity, and SiLU identities."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

U53 = 2.0 ** -53


def _exact_linear(x64, qw, s, z, N, K, G=128):
    """Exact rational value of sum_k x*s*(q-z) (all inputs are dyadic rationals)."""
    xf = [[Fraction(float(v)) for v in row] for row in x64]
    sf = [[Fraction(float(np.uint16(b).view(np.float16))) for b in row] for row in s]
    out = []
    for xr in xf:
        yr = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                byte = int(qw[n, k // 2])
                q = (byte >> 4) if (k % 2) else (byte & 15)
                acc += xr[k] * sf[n][k // G] * (q - int(z[n, k // G]))
            yr.append(acc)
        out.append(yr)
    return out


def test_whole_gemv_small_workload_against_exact_rationals():
    c = workloads.GEMV_SMALL
    w = workloads.weights(c["seed"], 0, c["N"], c["K"], *c["scale"])
    x = workloads.activations(c["seed"], 0, c["T"], c["K"], "f32")
    x64 = oracle.widen(x, "f32")
    y, S = oracle.linear(x64, w["qweight"], w["scales"], w["zeros"], c["N"], c["K"])
    ex = _exact_linear(x64, w["qweight"], w["scales"], w["zeros"], c["N"], c["K"])
    K = c["K"]
    for n in range(c["N"]):
        err = abs(Fraction(float(y[0, n])) - ex[0][n])
        assert err <= Fraction(2 * K * U53) * Fraction(float(S[0, n])), n


@pytest.mark.parametrize("T,N,K", [(3, 5, 128), (2, 7, 384), (1, 1, 256)])
def test_small_shapes_against_exact_rationals(T, N, K):
    w = workloads.weights(11, T * 100 + N, N, K, 0.002, 0.02)
    x64 = oracle.widen(workloads.activations(11, N, T, K, "bf16"), "bf16")
    y, S = oracle.linear(x64, w["qweight"], w["scales"], w["zeros"], N, K)
    ex = _exact_linear(x64, w["qweight"], w["scales"], w["zeros"], N, K)
    for t in range(T):
        for n in range(N):
            err = abs(Fraction(float(y[t, n])) - ex[t][n])
            assert err <= Fraction(2 * K * U53) * Fraction(float(S[t, n]))


@pytest.mark.parametrize("T,N,K,G", [(2, 5, 256, 64), (3, 4, 512, 256), (2, 3, 384, 384),
                                     (1, 6, 640, 640)])
def test_other_group_sizes_against_exact_rationals(T, N, K, G):
    # group sizes 64 and 256 (the FastLLM page's section 4.2 allows them beside
    # 128) and one group per row (G = K)
    w = workloads.weights(13, T * 100 + N + G, N, K, 0.002, 0.02, group=G)
    x64 = oracle.widen(workloads.activations(13, N + G, T, K, "bf16"), "bf16")
    y, S = oracle.linear(x64, w["qweight"], w["scales"], w["zeros"], N, K, group=G)
    ex = _exact_linear(x64, w["qweight"], w["scales"], w["zeros"], N, K, G)
    for t in range(T):
        for n in range(N):
            err = abs(Fraction(float(y[t, n])) - ex[t][n])
            assert err <= Fraction(2 * K * U53) * Fraction(float(S[t, n]))


def test_closed_form_ramp():
    # q_k = k mod 16, zero 8, scale 0.5, x_k = k+1 over one group of 128:
    # sum_k 0.5*(k mod 16 - 8)*(k+1) = 0.5 * sum_b (272 - 128 b), b = 0..7 = -704
    K = 128
    codes = np.arange(K) % 16
    qw = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8).reshape(1, K // 2)
    s = np.array([[np.float16(0.5).view(np.uint16)]], dtype=np.uint16)
    z = np.array([[8]], dtype=np.uint8)
    x = np.arange(1, K + 1, dtype=np.float64).reshape(1, K)
    y, S = oracle.linear(x, qw, s, z, 1, K)
    assert y[0, 0] == -704.0
    # S = 0.5 * sum |(k mod 16 - 8)| (k+1); |r-8| summed over r = 64 per block
    assert S[0, 0] == 0.5 * sum(abs(int(c) - 8) * (k + 1) for k, c in enumerate(codes))


def test_one_hot_activation_selects_a_weight_column():
    N, K = 6, 256
    w = workloads.weights(4, 4, N, K, 0.005, 0.02)
    W = oracle.dequant(w["qweight"], w["scales"], w["zeros"], N, K)
    for k in (0, 1, 127, 128, 200, 255):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y, _ = oracle.linear(x, w["qweight"], w["scales"], w["zeros"], N, K)
        assert np.array_equal(y[0], W[:, k])


def test_one_hot_weight_selects_an_activation():
    # all codes equal the zero point except (n0, k0) where q - z = 1 and the scale is 1
    N, K, n0, k0 = 4, 256, 2, 131
    qw = np.full((N, K // 2), 0x77, dtype=np.uint8)
    z = np.full((N, 2), 7, dtype=np.uint8)
    s = np.full((N, 2), 0x3C00, dtype=np.uint16)
    b = qw[n0, k0 // 2]
    qw[n0, k0 // 2] = (b & 0x0F) | (8 << 4) if k0 % 2 else (b & 0xF0) | 8
    x = np.random.default_rng(0).standard_normal((3, K))
    y, S = oracle.linear(x, qw, s, z, N, K)
    expect = np.zeros((3, N))
    expect[:, n0] = x[:, k0]
    assert np.array_equal(y, expect)
    assert np.array_equal(S, np.abs(expect))


def test_linearity_in_the_activation():
    N, K = 16, 512
    w = workloads.weights(6, 6, N, K, 0.005, 0.02)
    g = np.random.default_rng(1)
    x1, x2 = g.standard_normal((2, K)), g.standard_normal((2, K))
    y1, S1 = oracle.linear(x1, w["qweight"], w["scales"], w["zeros"], N, K)
    y2, S2 = oracle.linear(x2, w["qweight"], w["scales"], w["zeros"], N, K)
    y3, _ = oracle.linear(3 * x1 + x2, w["qweight"], w["scales"], w["zeros"], N, K)
    assert np.all(np.abs(y3 - (3 * y1 + y2)) <= 1e-12 * (3 * S1 + S2))


def test_doubling_every_scale_doubles_the_output():
    N, K = 8, 256
    w = workloads.weights(7, 7, N, K, 0.005, 0.02)
    s2 = (w["scales"].view(np.float16) * np.float16(2)).view(np.uint16)
    x = np.random.default_rng(2).standard_normal((1, K))
    y1, _ = oracle.linear(x, w["qweight"], w["scales"], w["zeros"], N, K)
    y2, _ = oracle.linear(x, w["qweight"], s2, w["zeros"], N, K)
    assert np.array_equal(y2, 2 * y1)


def test_matches_numpy_matmul_of_independent_dequant():
    N, K, T = 64, 1024, 4
    w = workloads.weights(8, 8, N, K, 0.005, 0.02)
    qw = w["qweight"]
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = qw & 15
    q[:, 1::2] = qw >> 4
    s = np.repeat(w["scales"].view(np.float16).astype(np.float64), 128, axis=1)
    z = np.repeat(w["zeros"].astype(np.int64), 128, axis=1)
    W = s * (q - z)
    x = np.random.default_rng(3).standard_normal((T, K))
    y, S = oracle.linear(x, qw, w["scales"], w["zeros"], N, K)
    assert np.all(np.abs(y - x @ W.T) <= 4 * K * U53 * S)
    assert np.allclose(S, np.abs(x) @ np.abs(W).T, rtol=1e-12)


def test_silu_identities():
    from scipy.special import expit
    for v in (-30.0, -3.5, -1.0, -1e-8, 0.0, 1e-8, 0.25, 1.0, 2.0, 7.0, 30.0):
        assert oracle.silu(v) == pytest.approx(v * expit(v), rel=1e-15, abs=1e-300)
        # silu(v) - silu(-v) = v * (sigmoid(v) + sigmoid(-v)) = v
        assert oracle.silu(v) - oracle.silu(-v) == pytest.approx(v, rel=1e-14, abs=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-20)


def test_gate_up_silu_rows_are_gate_then_up():
    I, K = 5, 256
    w = workloads.weights(9, 9, 2 * I, K, 0.005, 0.02)
    x = np.random.default_rng(4).standard_normal((2, K))
    y, S = oracle.linear(x, w["qweight"], w["scales"], w["zeros"], 2 * I, K)
    h, tol = oracle.gate_up_silu(x, w["qweight"], w["scales"], w["zeros"], I, K)
    from scipy.special import expit
    g, u = y[:, :I], y[:, I:]
    assert np.allclose(h, g * expit(g) * u, rtol=1e-14, atol=0)
    # the first-order tolerance is at least c*|silu(g)|*S_u and non-negative
    assert np.all(tol >= 2e-3 * np.abs(g * expit(g)) * S[:, I:] * (1 - 1e-12))
