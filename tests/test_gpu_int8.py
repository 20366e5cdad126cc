"""GPU parity of the 8-bit weights (flag QI4_INT8; the --quant-bit 8 option of
the FastLLM page, section 4.2, and the int8 weight type of the fastllm README):
pack/unpack and dequant_f32 bit for bit, qlinear_int8 within 2e-3 * sum|w*x| on
bf16 and float32 activations and the SiLU(gate)*up epilogue, the GPU quantizer
bit for bit against the oracle's 255-level quantizer, and the MoE layer with
8-bit experts through the decode and the prefill paths (including scales whose
high-plane value 16 * scale takes the prefill's plain-operand pass)."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

SC = (0.0003, 0.0012)   # 8-bit scales: |w| up to about 0.3, like the 4-bit workloads


def _w8(seed, tag, N, K, group=128, sc=SC):
    return workloads.weights(seed, tag, N, K, sc[0], sc[1], group=group, bits=8)


def _pack(w, flags, group):
    import ffn_int4_g128_amd as q
    return q.pack(to_dev(w["qweight"]), to_dev(w["scales"]), to_dev(w["zeros"]), w["N"], w["K"],
                  flags | q.QI4_INT8, group=group)


@pytest.mark.parametrize("group", [128, 64, 256, 0])
@pytest.mark.parametrize("N,K,flags", [(40, 768, 0), (48, 512, 1), (17, 1024, 0), (1, 128, 0)])
def test_pack_unpack_dequant_bit_exact(group, N, K, flags):
    import ffn_int4_g128_amd as q
    if group and K % group:
        pytest.skip("group does not divide K")
    w = _w8(91, N + K + group, N, K, group)
    packed = _pack(w, flags, group)
    assert packed.numel() == q.packed_bytes(N, K, flags | q.QI4_INT8, group)
    qw, sc, zr = q.unpack(packed, N, K, flags | q.QI4_INT8, group=group)
    assert np.array_equal(qw.cpu().numpy(), w["qweight"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), w["scales"])
    assert np.array_equal(zr.cpu().numpy(), w["zeros"])
    wd = q.dequant_f32(packed, N, K, flags | q.QI4_INT8, group=group).cpu().numpy()
    ref = oracle.dequant(w["qweight"], w["scales"], w["zeros"], N, K, group or K, bits=8)
    assert np.array_equal(wd.astype(np.float64), ref)


@pytest.mark.parametrize("group", [128, 64, 0])
@pytest.mark.parametrize("T,N,K,xd", [(1, 130, 768, "bf16"), (5, 64, 1024, "f32"),
                                      (33, 48, 512, "bf16"), (1, 4096, 4096, "bf16"),
                                      (32, 1000, 2048, "bf16"), (100, 80, 384, "bf16")])
def test_qlinear_int8(group, T, N, K, xd):
    import torch
    import ffn_int4_g128_amd as q
    if group and K % group:
        pytest.skip("group does not divide K")
    w = _w8(92, T * 7 + N + group, N, K, group)
    x = workloads.activations(92, N + K, T, K, xd)
    xt = bf16_dev(x) if xd == "bf16" else to_dev(x)
    y = q.qlinear(xt, _pack(w, 0, group), N, flags=q.QI4_INT8, out_dtype=torch.float32,
                  group=group)
    torch.cuda.synchronize()
    ref, S = oracle.linear(oracle.widen(x, xd), w["qweight"], w["scales"], w["zeros"], N, K,
                           group=group or K, bits=8)
    assert_within(to_f64(y), ref, oracle.C_TOL * S, f"int8 group {group} T{T} N{N} K{K} {xd}")


@pytest.mark.parametrize("group", [128, 64])
def test_qlinear_int8_silu_mul(group):
    import torch
    import ffn_int4_g128_amd as q
    T, I, K = 3, 40, 512
    w = _w8(93, group, 2 * I, K, group)
    x = workloads.activations(93, I, T, K, "bf16")
    y = q.qlinear(bf16_dev(x), _pack(w, q.QI4_PACK_GATEUP, group), 2 * I,
                  flags=q.QI4_PACK_GATEUP | q.QI4_INT8, out_dtype=torch.float32,
                  epilogue=q.QI4_EPI_SILU_MUL, group=group)
    torch.cuda.synchronize()
    h, tol = oracle.gate_up_silu(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"],
                                 I, K, group=group, bits=8)
    assert_within(to_f64(y), h, tol, f"int8 silu_mul group {group}")


def test_int4_call_rejects_an_8bit_matrix():
    import torch
    import ffn_int4_g128_amd as q
    w = _w8(94, 0, 16, 256)
    x = bf16_dev(workloads.activations(94, 0, 1, 256, "bf16"))
    y = torch.empty((1, 16), dtype=torch.float32, device="cuda")
    rc = q.lib().qlinear_int4(q._ptr(x), q.QI4_BF16, 1, 256, q._ptr(_pack(w, 0, 128)), 16, 128,
                              q.QI4_INT8, q._ptr(y), q.QI4_F32, 0, q._stream())
    assert rc == -7


@pytest.mark.parametrize("group", [128, 64, 256, 384, 0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_int8_bit_exact(group, dtype):
    import torch
    import ffn_int4_g128_amd as q
    N, K = 40, 1536
    g = np.random.default_rng(95 + group)
    w = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    w[0, :group or K] = 0.0
    w[1, :group or K] = 0.37
    w[2, :group or K] = -np.abs(w[2, :group or K])
    if dtype == "bf16":
        w = (torch.from_numpy(w).to(torch.bfloat16)).to(torch.float32).numpy()
        wt = torch.from_numpy(w).to(torch.bfloat16).cuda()
    else:
        wt = torch.from_numpy(w).cuda()
    qw, sc, zr = q.quantize(wt, group=group, flags=q.QI4_INT8)
    torch.cuda.synchronize()
    oqw, osc, ozr = oracle.quantize(w.astype(np.float64), group or K, bits=8)
    assert np.array_equal(qw.cpu().numpy(), oqw)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), osc)
    assert np.array_equal(zr.cpu().numpy(), ozr)


def _moe_check(E, H, I, k, T, group, seed, sc=SC, shared=True):
    import torch
    import ffn_int4_g128_amd as q
    ex = workloads.moe_experts(seed, 0, E, H, I, sc[0], sc[1], group=group, bits=8)
    sh = workloads.moe_shared(seed, 0, H, I, sc[0], sc[1], group=group, bits=8) if shared else None
    x = workloads.activations(seed + 1, T, T, H, "bf16")
    logits = workloads.logits_normal(seed + 2, T, T, E)
    mw = q.pack_moe(ex, sh, E, H, I, group=group, flags=q.QI4_INT8)
    out, ids, wts = q.moe_ffn(bf16_dev(x), mw, k, logits=to_dev(logits), return_routing=True)
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    return to_f64(out), oids, op, ex, sh, x


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("T", [1, 5, 33, 300])
def test_moe_int8(group, T):
    E, H, I, k = 8, 512, 256, 2
    out, oids, op, ex, sh, x = _moe_check(E, H, I, k, T, group, 96 + T)
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E, group=group, bits=8)
    assert_within(out, ref, tol, f"moe int8 group {group} T{T}")


@pytest.mark.parametrize("T", [12, 300])
def test_moe_int8_large_scales(T):
    # scales of 20..4000: the high plane's 16 * scale (320..64000) exceeds the
    # prefill's fast-pass range, so those tiles take the plain-operand pass
    E, H, I, k = 4, 256, 128, 2
    out, oids, op, ex, sh, x = _moe_check(E, H, I, k, T, 128, 97, sc=(20.0, 4000.0))
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E, bits=8)
    assert_within(out, ref, tol, f"moe int8 large scales T{T}")


@pytest.mark.parametrize("T", [8, 32])
def test_moe_int8_deepseek_expert_shape(T):
    # the DeepSeek-V3 expert shape (hidden 7168, intermediate 2048) with 16 experts,
    # top-8; the oracle checks four of the tokens
    E, H, I, k = 16, 7168, 2048, 8
    out, oids, op, ex, sh, x = _moe_check(E, H, I, k, T, 128, 98)
    sel = np.array([0, 1, T // 2, T - 1])
    ref, tol = oracle.moe(oracle.widen(x, "bf16")[sel], oids[sel], op[sel], ex, sh, H, I, E, bits=8)
    assert_within(out[sel], ref, tol, f"moe int8 deepseek shape T{T}")
