"""GPU parity of qlinear_int4_g128 against the oracle: the small GEMV, ragged and
multi-tile shapes, the fused SiLU(gate)*up epilogue, the Llama-7B-shaped decode
stack and the skinny decode sweep (every token at full size), plus edge cases.
Shapes with more than 16 rows and rows too long for LDS (T = 33, 47, 64; the
SiLU cases at T = 17 and 40) take the row-major activation loads.
Tolerance: |gpu - oracle| <= 2e-3 * sum_k |w*x| per output element; for the
fused epilogue its first-order propagation through SiLU(g)*u."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, pack_canonical, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _run(w, x, x_dtype, out_dtype, flags=0, epi=0):
    import torch
    import ffn_int4_g128_amd as q
    packed = pack_canonical(w, flags)
    xt = bf16_dev(x) if x_dtype == "bf16" else to_dev(x)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    y = q.qlinear(xt, packed, w["N"], flags=flags, out_dtype=od, epilogue=epi)
    torch.cuda.synchronize()
    return to_f64(y)


def test_gemv_small_f32():
    c = workloads.GEMV_SMALL
    w = workloads.weights(c["seed"], 0, c["N"], c["K"], *c["scale"])
    x = workloads.activations(c["seed"], 0, c["T"], c["K"], "f32")
    got = _run(w, x, "f32", "f32")
    ref, S = oracle.linear(oracle.widen(x, "f32"), w["qweight"], w["scales"], w["zeros"],
                           c["N"], c["K"])
    assert_within(got, ref, oracle.C_TOL * S, "gemv_k256_n128_f32")


@pytest.mark.parametrize("T,N,K,xd,od", [
    (1, 128, 256, "bf16", "f32"), (3, 17, 128, "bf16", "f32"), (16, 130, 384, "bf16", "bf16"),
    (17, 64, 512, "bf16", "f32"), (33, 48, 1024, "bf16", "f32"), (5, 200, 2048, "f32", "f32"),
    (7, 33, 256, "f32", "bf16"), (1, 4096, 4096, "bf16", "bf16"), (64, 96, 640, "bf16", "f32"),
    (47, 4112, 1536, "bf16", "bf16"), (1, 48, 32768, "bf16", "f32"),
    (3, 40, 20480, "f32", "bf16"), (24, 32, 16384, "bf16", "f32")])
def test_shapes(T, N, K, xd, od):
    w = workloads.weights(31, T * 1000 + N, N, K, 0.005, 0.02)
    x = workloads.activations(31, N + K, T, K, xd)
    got = _run(w, x, xd, od)
    ref, S = oracle.linear(oracle.widen(x, xd), w["qweight"], w["scales"], w["zeros"], N, K)
    assert_within(got, ref, oracle.C_TOL * S, f"T{T} N{N} K{K} {xd}->{od}")


@pytest.mark.parametrize("T,I,K,od", [(1, 64, 256, "f32"), (4, 24, 128, "f32"),
                                      (19, 40, 384, "bf16"), (1, 11008, 4096, "bf16"),
                                      (40, 64, 2048, "f32"), (17, 1000, 1024, "bf16")])
def test_silu_mul_epilogue(T, I, K, od):
    import ffn_int4_g128_amd as q
    w = workloads.weights(41, I + T, 2 * I, K, 0.005, 0.02)
    x = workloads.activations(41, I * 7 + K, T, K, "bf16")
    got = _run(w, x, "bf16", od, flags=q.QI4_PACK_GATEUP, epi=q.QI4_EPI_SILU_MUL)
    h, tol = oracle.gate_up_silu(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"],
                                 I, K)
    assert_within(got, h, tol, f"silu_mul T{T} I{I} K{K} ->{od}")


def test_gateup_packing_without_epilogue_keeps_row_order():
    import ffn_int4_g128_amd as q
    T, I, K = 3, 40, 256
    w = workloads.weights(42, 1, 2 * I, K, 0.005, 0.02)
    x = workloads.activations(42, 2, T, K, "bf16")
    got = _run(w, x, "bf16", "f32", flags=q.QI4_PACK_GATEUP)
    ref, S = oracle.linear(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"], 2 * I, K)
    assert_within(got, ref, oracle.C_TOL * S, "gateup packing, no epilogue")


def test_llama7b_decode_stack_each_linear():
    """Each linear of the Llama-7B-shaped stack at T=1 with its own fresh input."""
    import ffn_int4_g128_amd as q
    c = workloads.LLAMA7B_STACK
    for li, (name, K, N, epi) in enumerate(c["linears"]):
        w = workloads.weights(c["seed"], 10 + li, N, K, *c["scale"])
        x = workloads.activations(c["seed"], 20 + li, c["T"], K, "bf16")
        if epi == "silu_mul":
            got = _run(w, x, "bf16", "bf16", flags=q.QI4_PACK_GATEUP, epi=q.QI4_EPI_SILU_MUL)
            ref, tol = oracle.gate_up_silu(oracle.widen(x, "bf16"), w["qweight"], w["scales"],
                                           w["zeros"], N // 2, K)
        else:
            got = _run(w, x, "bf16", "bf16")
            ref, S = oracle.linear(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"],
                                   N, K)
            tol = oracle.C_TOL * S
        assert_within(got, ref, tol, f"llama7b {name} K{K} N{N}")


@pytest.mark.parametrize("K,N", workloads.SKINNY_SWEEP["shapes"])
@pytest.mark.parametrize("T", workloads.SKINNY_SWEEP["T"])
def test_skinny_sweep_every_token(K, N, T):
    """Full-size launch, in the launch shape the benchmark times; the oracle
    checks every token and every column."""
    c = workloads.SKINNY_SWEEP
    w = workloads.weights(c["seed"], K, N, K, *c["scale"])
    x = workloads.activations(c["seed"], 100 + T, T, K, "bf16", scale=c["x_scale"])
    got = _run(w, x, "bf16", "bf16")
    ref, S = oracle.linear(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"], N, K)
    assert_within(got, ref, oracle.C_TOL * S, f"skinny K{K} N{N} T{T} all rows")


def test_all_zero_weights_give_exact_zero():
    """q == zero everywhere: every dequantized weight is 0, so is every output."""
    T, N, K = 5, 40, 512
    w = workloads.weights(51, 0, N, K, 0.005, 0.02)
    z = w["zeros"]
    for g in range(K // 128):
        b = (z[:, g] | (z[:, g] << 4)).astype(np.uint8)
        w["qweight"][:, 64 * g:64 * (g + 1)] = b[:, None]
    x = workloads.activations(51, 1, T, K, "bf16")
    got = _run(w, x, "bf16", "f32")
    assert np.all(got == 0.0)


def test_zero_scale_rows_and_empty_batch():
    import torch
    import ffn_int4_g128_amd as q
    T, N, K = 4, 32, 256
    w = workloads.weights(52, 0, N, K, 0.005, 0.02)
    w["scales"][5:9] = 0
    x = workloads.activations(52, 1, T, K, "bf16")
    got = _run(w, x, "bf16", "f32")
    assert np.all(got[:, 5:9] == 0.0)
    packed = pack_canonical(w)
    empty = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    y = q.qlinear(empty, packed, N)
    assert y.shape == (0, N)


@pytest.mark.parametrize("T", [9, 40])
def test_repeat_is_deterministic(T):
    import torch
    import ffn_int4_g128_amd as q
    N, K = 1000, 4096
    w = workloads.weights(53, 0, N, K, 0.005, 0.02)
    x = bf16_dev(workloads.activations(53, 1, T, K, "bf16"))
    packed = pack_canonical(w)
    a = q.qlinear(x, packed, N, out_dtype=torch.float32)
    b = q.qlinear(x, packed, N, out_dtype=torch.float32)
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,N,K", [(1, 80, 2048), (3, 48, 1024), (17, 40, 512), (2, 4096, 4096),
                                   (20, 64, 2048)])
def test_blocks_of_very_different_magnitude(T, N, K):
    """Each 128-wide block of a row carries its own power of two (2^-24 .. 2^+24,
    a different one per block and row), so the rows' fp16 conversion must use
    one exponent per (row, block): a factor applied to the wrong block or row
    is off by many orders of magnitude against 2e-3 * sum|w*x|.  Few short rows
    are converted into LDS by each workgroup, T = 20 x 2048 in registers."""
    w = workloads.weights(61, T * 100 + K, N, K, 0.005, 0.02)
    x = workloads.activations(61, N + K, T, K, "bf16")
    xf = workloads.bf16_bits_to_f32(x).reshape(T, K // 128, 128)
    e = (np.arange(T)[:, None] * 5 + np.arange(K // 128)[None, :] * 11) % 49 - 24
    x = workloads.f32_to_bf16_bits((xf * np.exp2(e)[:, :, None]).reshape(T, K).astype(np.float32))
    got = _run(w, x, "bf16", "f32")
    ref, S = oracle.linear(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"], N, K)
    assert_within(got, ref, oracle.C_TOL * S, f"wide-range blocks T{T} N{N} K{K}")
