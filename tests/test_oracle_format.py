"""Pins of the oracle's format handling: nibble order, binary16 decoding,
dequantization identities, and the byte cost stated by the pages."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLD, "page_facts.json")) as f:
        return json.load(f)


def test_unpack_every_byte_value():
    # one row, K = 512: byte b holds k = 2b (low nibble) and k = 2b+1 (high nibble)
    qw = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = oracle.unpack(qw, 1, 512)
    for b in range(256):
        hi, lo = divmod(b, 16)
        assert q[0, 2 * b] == lo and q[0, 2 * b + 1] == hi


def test_unpack_rows_do_not_mix():
    qw = np.array([[0x21, 0x43], [0x65, 0x87]], dtype=np.uint8)
    q = oracle.unpack(qw, 2, 4)
    assert q.tolist() == [[1, 2, 3, 4], [5, 6, 7, 8]]


def test_f16_decode_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_encode_rounds_like_numpy():
    g = np.random.default_rng(5)
    vals = np.concatenate([g.uniform(-70000, 70000, 2000), g.uniform(-1e-4, 1e-4, 2000),
                           g.uniform(0.001, 0.03, 2000),
                           # exact ties between neighbouring binary16 values
                           (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -10,
                           [0.0, -0.0, 65504.0, 65519.99, 65520.0, 2 ** -24, 2 ** -25, 3 * 2 ** -26]])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _rand_w(N, K, seed=0, G=128):
    w = workloads.weights(seed, 9, N, K, 0.005, 0.02, G)
    return w["qweight"], w["scales"], w["zeros"]


def test_dequant_zero_when_q_equals_zero_point():
    N, K = 4, 256
    qw, s, _ = _rand_w(N, K)
    z = np.full((N, K // 128), 9, dtype=np.uint8)
    qw[:] = 0x99
    w = oracle.dequant(qw, s, z, N, K)
    assert np.all(w == 0.0)


def test_dequant_equal_codes_give_constant_group():
    N, K = 3, 384
    qw, s, z = _rand_w(N, K, seed=1)
    qw[:] = 0x55  # every code is 5
    w = oracle.dequant(qw, s, z, N, K)
    for n in range(N):
        for g in range(K // 128):
            blk = w[n, 128 * g:128 * (g + 1)]
            assert np.all(blk == blk[0])
            assert blk[0] == np.float64(np.uint16(s[n, g]).view(np.float16)) * (5 - int(z[n, g]))


def test_dequant_unit_scale_is_code_minus_zero():
    N, K = 2, 256
    qw, _, _ = _rand_w(N, K, seed=2)
    one = np.full((N, 2), 0x3C00, dtype=np.uint16)  # binary16 1.0
    z0 = np.zeros((N, 2), dtype=np.uint8)
    z8 = np.full((N, 2), 8, dtype=np.uint8)
    q = oracle.unpack(qw, N, K).astype(np.float64)
    assert np.array_equal(oracle.dequant(qw, one, z0, N, K), q)
    assert np.array_equal(oracle.dequant(qw, one, z8, N, K), q - 8)


def test_dequant_group_boundary_and_row_indexing():
    # row n, group g gets scale 2^(n*2+g) and zero g; every code is 3
    N, K = 2, 256
    qw = np.full((N, K // 2), 0x33, dtype=np.uint8)
    s = np.array([[0x3C00, 0x4000], [0x4400, 0x4800]], dtype=np.uint16)  # 1, 2, 4, 8
    z = np.array([[0, 1], [0, 1]], dtype=np.uint8)
    w = oracle.dequant(qw, s, z, N, K)
    assert np.all(w[0, :128] == 3.0) and np.all(w[0, 128:] == 4.0)
    assert np.all(w[1, :128] == 12.0) and np.all(w[1, 128:] == 16.0)


def test_dequant_group_sizes_relate():
    # a matrix quantized with 64-wide groups whose neighbours share scale and zero
    # is the 128-wide matrix with those values; 256-wide and per-row (one group
    # per row, G = K) groups are 128-wide ones with repeated values
    N, K = 3, 512
    g = np.random.default_rng(5)
    qw = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s128 = g.uniform(0.01, 0.02, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    z128 = g.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    w128 = oracle.dequant(qw, s128, z128, N, K)
    assert np.array_equal(oracle.dequant(qw, np.repeat(s128, 2, axis=1), np.repeat(z128, 2, axis=1),
                                         N, K, group=64), w128)
    s256, z256 = s128[:, ::2], z128[:, ::2]
    assert np.array_equal(oracle.dequant(qw, s256, z256, N, K, group=256),
                          oracle.dequant(qw, np.repeat(s256, 2, axis=1), np.repeat(z256, 2, axis=1),
                                         N, K))
    sr, zr = s128[:, :1], z128[:, :1]
    assert np.array_equal(oracle.dequant(qw, sr, zr, N, K, group=K),
                          oracle.dequant(qw, np.repeat(sr, 4, axis=1), np.repeat(zr, 4, axis=1), N, K))
    # and a 64-wide group boundary really splits a 128-wide block
    s64 = np.array([[0x3C00, 0x4000]], dtype=np.uint16)      # 1, 2
    z64 = np.array([[0, 1]], dtype=np.uint8)
    w = oracle.dequant(np.full((1, 64), 0x33, dtype=np.uint8), s64, z64, 1, 128, group=64)
    assert np.all(w[0, :64] == 3.0) and np.all(w[0, 64:] == 4.0)


def test_dequant_exact_in_fp32_for_workload_scales():
    # s*(q-z) for every binary16 scale of the workload range and every q-z is exact in
    # binary32: the product of an 11-bit and a 5-bit integer significand has <= 16 bits
    lo, hi = np.float16(0.002).view(np.uint16), np.float16(0.02).view(np.uint16)
    bits = np.arange(lo, hi + 1, dtype=np.uint16)
    s64 = bits.view(np.float16).astype(np.float64)
    for m in range(-15, 16):
        prod = s64 * m
        assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)


def test_format_byte_cost_matches_page_size_fact():
    f = _facts()
    G, bits = f["group_size"]["value"], f["bits_per_code"]["value"]
    assert G == workloads.GROUP and bits == 4
    n = f["n_weights_7b"]["value"]
    per_w = workloads.packed_weight_bytes(1)
    assert per_w == pytest.approx((G * bits / 8 + 2 + 0.5) / G)
    total = n * per_w
    # the page's ~3.8 GB includes unquantized tensors; the codes+scales+zeros must
    # fit under it and be well below the 14 GB of FP16
    assert 3.3e9 < total <= f["int4_7b_model_bytes_approx"]["value"]
    assert f["fp16_7b_weight_bytes"]["value"] == pytest.approx(2 * n)
    # the bandwidth argument: time per token = bytes read / bandwidth
    t = f["fp16_7b_weight_bytes"]["value"] / f["ddr4_2666_bandwidth_bytes_per_s"]["value"]
    assert t == pytest.approx(f["fp16_7b_read_time_s"]["value"])


def test_bf16_rounding_of_inputs_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(100000, dtype=np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]  # exact ties
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
