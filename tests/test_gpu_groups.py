"""GPU parity of the group-size variants -- 64-wide and 256-wide groups (the
FastLLM page's section 4.2 allows them beside 128) and one group per row (the
plain int4 of the fastllm README, group_size 0): pack/unpack and dequant_f32 bit
for bit, qlinear within 2e-3 * sum|w*x|, the GPU quantizer bit for bit against
the oracle's, and the MoE layer through the decode and the prefill paths."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

GROUPS = [64, 256, 0]


def _pack(w, flags, group):
    import ffn_int4_g128_amd as q
    return q.pack(to_dev(w["qweight"]), to_dev(w["scales"]), to_dev(w["zeros"]), w["N"], w["K"],
                  flags, group=group)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("N,K,flags", [(40, 768, 0), (48, 512, 1), (17, 1024, 0)])
def test_pack_unpack_dequant_bit_exact(group, N, K, flags):
    import ffn_int4_g128_amd as q
    w = workloads.weights(81, N + K + group, N, K, 0.005, 0.02, group=group)
    packed = _pack(w, flags, group)
    qw, sc, zr = q.unpack(packed, N, K, flags, group=group)
    assert np.array_equal(qw.cpu().numpy(), w["qweight"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), w["scales"])
    assert np.array_equal(zr.cpu().numpy(), w["zeros"])
    wd = q.dequant_f32(packed, N, K, flags, group=group).cpu().numpy().astype(np.float64)
    ref = oracle.dequant(w["qweight"], w["scales"], w["zeros"], N, K, group or K)
    assert np.array_equal(wd, ref)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("T,N,K,xd", [(1, 130, 768, "bf16"), (5, 64, 1024, "f32"),
                                      (33, 48, 512, "bf16"), (1, 4096, 4096, "bf16")])
def test_qlinear(group, T, N, K, xd):
    import torch
    import ffn_int4_g128_amd as q
    w = workloads.weights(82, T * 7 + N + group, N, K, 0.005, 0.02, group=group)
    x = workloads.activations(82, N + K, T, K, xd)
    xt = bf16_dev(x) if xd == "bf16" else to_dev(x)
    y = q.qlinear(xt, _pack(w, 0, group), N, out_dtype=torch.float32, group=group)
    torch.cuda.synchronize()
    ref, S = oracle.linear(oracle.widen(x, xd), w["qweight"], w["scales"], w["zeros"], N, K,
                           group=group or K)
    assert_within(to_f64(y), ref, oracle.C_TOL * S, f"group {group} T{T} N{N} K{K} {xd}")


@pytest.mark.parametrize("group", GROUPS)
def test_qlinear_silu_mul(group):
    import torch
    import ffn_int4_g128_amd as q
    T, I, K = 3, 40, 512
    w = workloads.weights(83, group, 2 * I, K, 0.005, 0.02, group=group)
    x = workloads.activations(83, I, T, K, "bf16")
    y = q.qlinear(bf16_dev(x), _pack(w, q.QI4_PACK_GATEUP, group), 2 * I,
                  flags=q.QI4_PACK_GATEUP, out_dtype=torch.float32, epilogue=q.QI4_EPI_SILU_MUL,
                  group=group)
    torch.cuda.synchronize()
    h, tol = oracle.gate_up_silu(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"],
                                 I, K, group=group or K)
    assert_within(to_f64(y), h, tol, f"silu_mul group {group}")


@pytest.mark.parametrize("group", [64, 256, 512, 384, 0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(group, dtype):
    import torch
    import ffn_int4_g128_amd as q
    N, K = 40, 1536
    g = np.random.default_rng(84 + group)
    w = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    w[0, :group or K] = 0.0
    w[1, :group or K] = 0.37
    if dtype == "bf16":
        w = (torch.from_numpy(w).to(torch.bfloat16)).to(torch.float32).numpy()
        wt = torch.from_numpy(w).to(torch.bfloat16).cuda()
    else:
        wt = torch.from_numpy(w).cuda()
    qw, sc, zr = q.quantize(wt, group=group)
    torch.cuda.synchronize()
    oqw, osc, ozr = oracle.quantize(w.astype(np.float64), group or K)
    assert np.array_equal(qw.cpu().numpy(), oqw)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), osc)
    assert np.array_equal(zr.cpu().numpy(), ozr)


@pytest.mark.parametrize("group", [64, 256, 0])
@pytest.mark.parametrize("T", [5, 300])
def test_moe(group, T):
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 512, 256, 2
    ex = workloads.moe_experts(85, 0, E, H, I, 0.005, 0.02, group=group)
    sh = workloads.moe_shared(85, 0, H, I, 0.005, 0.02, group=group)
    x = workloads.activations(86, T, T, H, "bf16")
    logits = workloads.logits_normal(87, T, T, E)
    mw = q.pack_moe(ex, sh, E, H, I, group=group)
    out, ids, wts = q.moe_ffn(bf16_dev(x), mw, k, logits=to_dev(logits), return_routing=True)
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E, group=group)
    assert_within(to_f64(out), ref, tol, f"moe group {group} T{T}")
