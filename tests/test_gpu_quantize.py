"""GPU load-time quantizer against the oracle's reference quantizer: codes, scales
and zero points bit for bit, on seeded weights (float32 and bf16) and on groups
built to hit every decision the quantizer takes: an all-zero group, constant
groups of either sign, all-negative and all-positive groups, weights exactly
halfway between two code levels (ties to even), scales that round to binary16
subnormals, to the largest binary16 values and past them, and a group whose
scale rounds to zero."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _gpu(w, dtype):
    import torch
    import ffn_int4_g128_amd as q
    t = torch.from_numpy(np.ascontiguousarray(w.astype(np.float32))).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    qw, s, z = q.quantize(t)
    torch.cuda.synchronize()
    return qw.cpu().numpy(), s.cpu().numpy().view(np.uint16), z.cpu().numpy()


def _check(w, dtype, what):
    wq = w.astype(np.float32)
    if dtype == "bf16":
        wq = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(wq))
    rq, rs, rz = oracle.quantize(wq.astype(np.float64))
    gq, gs, gz = _gpu(wq, dtype)
    assert np.array_equal(gs, rs), f"{what}: scales differ at {np.argwhere(gs != rs)[:5]}"
    assert np.array_equal(gz, rz), f"{what}: zeros differ at {np.argwhere(gz != rz)[:5]}"
    assert np.array_equal(gq, rq), f"{what}: codes differ at {np.argwhere(gq != rq)[:5]}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (64, 4096)])
def test_quantize_random_matches_oracle(N, K, dtype):
    g = np.random.default_rng([21, N, K])
    w = (g.standard_normal((N, K)) * g.uniform(0.001, 0.1, size=(N, 1))).astype(np.float32)
    _check(w, dtype, f"random {N}x{K} {dtype}")


def _edge_groups():
    g = np.random.default_rng(23)
    rows = []
    rows.append(np.zeros(128))                                  # all zero: scale 1.0, zero 0
    rows.append(np.full(128, 0.37))                             # constant positive
    rows.append(np.full(128, -2.5))                             # constant negative
    rows.append(-np.abs(g.standard_normal(128)))                # all negative
    rows.append(np.abs(g.standard_normal(128)) * 3)             # all positive
    # ties: range [-0.75, 0.75] -> scale 0.1 (not exact in binary16); then weights
    # placed exactly halfway between levels of the stored scale
    s = float(np.float16(0.1))
    lv = np.arange(-7, 8) * s
    row = np.concatenate([lv + 0.5 * s, lv - 0.5 * s])[:128]
    row = np.pad(row, (0, 128 - row.size), constant_values=0.0)
    row[0], row[1] = -7.5 * s, 7.5 * s
    rows.append(row)
    rows.append(g.standard_normal(128) * 1e-6)                  # subnormal scale
    rows.append(g.standard_normal(128) * 1e-9)                  # scale rounds to 0 -> 1.0
    rows.append(np.linspace(-5.0e5, 5.0e5, 128))                # scale past binary16: inf
    rows.append(np.linspace(-9.8e5 / 2, 9.8e5 / 2, 128) / 1e1)  # large finite scale
    return np.stack(rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_edge_groups_match_oracle(dtype):
    w = _edge_groups().astype(np.float32)
    w = np.concatenate([w, w[:, ::-1]], axis=1)    # K = 256: two groups per row
    _check(w, dtype, f"edge groups {dtype}")


def test_quantize_pack_linear_round_trip():
    """quantize -> pack -> qlinear equals the oracle linear on the same codes."""
    import torch
    import ffn_int4_g128_amd as q
    from tests._gpu import assert_within, to_f64
    g = np.random.default_rng(24)
    N, K, T = 96, 512, 3
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    qw, s, z = q.quantize(torch.from_numpy(w).cuda())
    packed = q.pack(qw, s, z, N, K)
    x = workloads.activations(25, 0, T, K, "f32")
    y = q.qlinear(torch.from_numpy(x).cuda(), packed, N)
    torch.cuda.synchronize()
    ref, S = oracle.linear(oracle.widen(x, "f32"), qw.cpu().numpy(),
                           s.cpu().numpy().view(np.uint16), z.cpu().numpy(), N, K)
    assert_within(to_f64(y), ref, oracle.C_TOL * S, "quantize -> pack -> qlinear")
