"""Pins of the oracle's 8-bit weights (the --quant-bit 8 variant of the format:
one byte per code, q and zero in 0..255, the same groups and binary16 scales).

Independent anchors: the already-pinned 4-bit oracle (an 8-bit matrix whose codes
and zeros are below 16 is the same matrix; and any 8-bit matrix is the sum of
two 4-bit matrices, one per nibble, exactly), closed forms over all 256 codes,
exact rational brute force, and the page's memory figures for 4- and 8-bit 7B
models."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

U53 = 2.0 ** -53
_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def _w8(N, K, seed=0, G=128, lo=0.0005, hi=0.002):
    w = workloads.weights(seed, 21, N, K, lo, hi, G, bits=8)
    return w["qweight"], w["scales"], w["zeros"]


def _pack4(q):
    """Nibble-pack codes 0..15 [N][K] into the 4-bit canonical layout (even k low)."""
    q = q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def _f16(v):
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def test_unpack8_returns_the_bytes():
    qw, _, _ = _w8(3, 256)
    assert np.array_equal(oracle.unpack(qw, 3, 256, bits=8), qw)


def test_codes_below_16_give_the_4bit_matrix():
    N, K = 4, 384
    g = np.random.default_rng(3)
    q = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = _f16(g.uniform(0.005, 0.02, size=(N, K // 128)))
    z = g.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    assert np.array_equal(oracle.dequant(q, s, z, N, K, bits=8), oracle.dequant(_pack4(q), s, z, N, K))
    x = oracle.widen(workloads.activations(3, 1, 2, K, "bf16"), "bf16")
    y8, S8 = oracle.linear(x, q, s, z, N, K, bits=8)
    y4, S4 = oracle.linear(x, _pack4(q), s, z, N, K)
    assert np.array_equal(y8, y4) and np.array_equal(S8, S4)


@pytest.mark.parametrize("G", [128, 64, 256])
def test_nibble_split_identity(G):
    # s*(q - z) = 16s*(q>>4 - z>>4) + s*(q&15 - z&15): two 4-bit matrices, exactly
    N, K = 5, 512
    q, s, z = _w8(N, K, seed=G, G=G)
    s16 = _f16(s.view(np.float16).astype(np.float64) * 16)   # exact: power-of-two factor
    hi = oracle.dequant(_pack4(q >> 4), s16, z >> 4, N, K, G)
    lo = oracle.dequant(_pack4(q & 15), s, z & 15, N, K, G)
    assert np.array_equal(oracle.dequant(q, s, z, N, K, G, bits=8), hi + lo)


def test_closed_forms_over_all_codes():
    # one row holding every code 0..255 with unit scale: w = q - z for each zero
    K = 256
    q = np.arange(256, dtype=np.uint8).reshape(1, K)
    one = _f16([[1.0, 1.0]])
    for zv in (0, 1, 128, 200, 255):
        z = np.full((1, 2), zv, dtype=np.uint8)
        w = oracle.dequant(q, one, z, 1, K, bits=8)
        assert np.array_equal(w[0], np.arange(256, dtype=np.float64) - zv)
    # q == z gives 0; equal codes give a constant group
    qz = np.full((2, K), 77, dtype=np.uint8)
    s = _f16([[0.01, 0.02], [0.03, 0.04]])
    assert np.all(oracle.dequant(qz, s, np.full((2, 2), 77, dtype=np.uint8), 2, K, bits=8) == 0)
    w = oracle.dequant(qz, s, np.full((2, 2), 13, dtype=np.uint8), 2, K, bits=8)
    for n in range(2):
        for gi in range(2):
            blk = w[n, 128 * gi:128 * (gi + 1)]
            assert np.all(blk == float(s[n, gi:gi + 1].view(np.float16)[0]) * 64)


def _exact_linear8(x64, q, s, z, N, K, G):
    xf = [[Fraction(float(v)) for v in row] for row in x64]
    sf = [[Fraction(float(np.uint16(b).view(np.float16))) for b in row] for row in s]
    return [[sum((xr[k] * sf[n][k // G] * (int(q[n, k]) - int(z[n, k // G])) for k in range(K)),
                 Fraction(0)) for n in range(N)] for xr in xf]


@pytest.mark.parametrize("T,N,K,G", [(2, 3, 256, 128), (1, 4, 256, 64), (2, 2, 512, 256)])
def test_linear8_against_exact_rationals(T, N, K, G):
    q, s, z = _w8(N, K, seed=T * 10 + N, G=G)
    x64 = oracle.widen(workloads.activations(12, N, T, K, "bf16"), "bf16")
    y, S = oracle.linear(x64, q, s, z, N, K, G, bits=8)
    ex = _exact_linear8(x64, q, s, z, N, K, G)
    for t in range(T):
        for n in range(N):
            assert abs(Fraction(float(y[t, n])) - ex[t][n]) <= Fraction(2 * K * U53) * Fraction(float(S[t, n]))


def test_gate_up8_rows_are_gate_then_up():
    I, K = 3, 256
    q, s, z = _w8(2 * I, K, seed=4)
    x64 = oracle.widen(workloads.activations(4, 2, 2, K, "bf16"), "bf16")
    gu, _ = oracle.linear(x64, q, s, z, 2 * I, K, bits=8)
    h, _ = oracle.gate_up_silu(x64, q, s, z, I, K, bits=8)
    for t in range(2):
        for i in range(I):
            assert h[t, i] == oracle.silu(gu[t, i]) * gu[t, I + i]


def test_moe8_top1_and_small_codes():
    # top-1 with weight 1 reduces to one expert's FFN; and 8-bit experts whose codes
    # are below 16 give the 4-bit layer (checks the per-expert code strides)
    E, H, I = 3, 256, 128
    g = np.random.default_rng(8)
    ex = workloads.moe_experts(8, 0, E, H, I, 0.005, 0.02, bits=8)
    x64 = oracle.widen(workloads.activations(8, 3, 2, H, "bf16"), "bf16")
    ids = np.array([[2], [1]], dtype=np.int32)
    p = np.ones((2, 1))
    out, _ = oracle.moe(x64, ids, p, ex, None, H, I, E, bits=8)
    for t in range(2):
        e = ids[t, 0]
        h, _ = oracle.gate_up_silu(x64[t:t + 1], ex["gu_q"][e], ex["gu_s"][e], ex["gu_z"][e], I, H, bits=8)
        y, _ = oracle.linear(h, ex["dn_q"][e], ex["dn_s"][e], ex["dn_z"][e], H, I, bits=8)
        assert np.array_equal(out[t], y[0])
    small = {k: (v & 15 if k.endswith(("_q", "_z")) else v) for k, v in ex.items()}
    four = dict(small, gu_q=np.stack([_pack4(m) for m in small["gu_q"]]),
                dn_q=np.stack([_pack4(m) for m in small["dn_q"]]))
    ids2 = g.permutation(E)[:2].reshape(1, 2).astype(np.int32).repeat(2, axis=0)
    p2 = np.array([[0.25, 0.75], [0.5, 0.5]])
    o8, t8 = oracle.moe(x64, ids2, p2, small, None, H, I, E, bits=8)
    o4, t4 = oracle.moe(x64, ids2, p2, four, None, H, I, E)
    assert np.array_equal(o8, o4) and np.array_equal(t8, t4)


@pytest.mark.parametrize("G", [128, 64, 256])
def test_quantizer8_error_bound_and_round_trip(G):
    g = np.random.default_rng(19)
    w = g.standard_normal((6, 512)) * 0.05
    w[0, :G] = 0.0
    w[1, :G] = 0.37
    w[2, :G] = -np.abs(w[2, :G])
    qw, s, z = oracle.quantize(w, G, bits=8)
    assert qw.shape == (6, 512) and qw.max() > 200   # the 8-bit range is used
    wd = oracle.dequant(qw, s, z, 6, 512, G, bits=8)
    sc = np.repeat(s.view(np.float16).astype(np.float64), G, axis=1)
    assert np.all(np.abs(w - wd) <= sc * (0.5 + 1e-3) + 1e-12)
    assert np.all(wd[0, :G] == 0.0)
    zz = np.repeat(z.astype(np.int64), G, axis=1)
    assert np.array_equal(np.clip(np.rint(wd / sc) + zz, 0, 255), qw.astype(np.int64))
    # 255 levels instead of 15: the scales are about 15/255 of the 4-bit ones
    _, s4, _ = oracle.quantize(w, G)
    r = s.view(np.float16).astype(np.float64)[3:] / s4.view(np.float16).astype(np.float64)[3:]
    assert np.all(np.abs(r - 15 / 255) < 2e-3)


def test_format_cost_matches_page_memory_figures():
    facts = json.load(open(_GOLDEN))
    n = facts["n_weights_7b"]["value"]
    m4, m8 = facts["mem_7b_4bit_bytes"]["value"], facts["mem_7b_8bit_bytes"]["value"]
    # the two runs differ only in the weights: the difference is the weight-size gap
    gap = n * (workloads.packed_weight_bytes(1, 128, 8) - workloads.packed_weight_bytes(1, 128, 4))
    assert abs(gap - (m8 - m4)) <= 0.2 * (m8 - m4)
