"""GPU parity on inputs built to expose cancellation in the kernels' sums.

The layer computes y = sum_k x_k * s * (q_k - zero).  When almost every code of
a group sits on its zero point, the true result is a handful of small products
while the activations of the group can be large (an outlier).  A kernel that
forms the group's sum as (sum x * (c + q)) - (sum x * (c + zero)) for a large
offset c loses the small difference in the rounding of the two large sums; the
tolerance 2e-3 * sum|w*x| (per output element) does not allow that.  These
cases are checked element by element on every kernel family: the decode GEMM
(bf16 and fp32 activations, plain and SiLU(gate)*up epilogue) and the MoE layer
on its decode and prefill paths.  Also: a row holding an inf or NaN leaves
every other row's result as the oracle gives it."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, pack_canonical, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _pack_codes(q: np.ndarray) -> np.ndarray:
    """[N][K] codes 0..15 -> canonical bytes [N][K/2], even k in the low nibble."""
    q = q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def sparse_weights(seed: int, N: int, K: int, off_per_row, group: int = 128) -> dict:
    """Codes equal to their group's zero point except `off_per_row[n]` codes of
    row n, which differ from it by +-1 (or +-7 for every third of them); scales
    U[0.005, 0.02].  Row 0 has no code off its zero point."""
    g = np.random.default_rng([seed, N, K])
    G = K // group
    zeros = g.integers(0, 16, size=(N, G), dtype=np.uint8)
    q = np.repeat(zeros.astype(np.int64), group, axis=1)
    for n in range(N):
        for i, k in enumerate(g.choice(K, size=off_per_row[n], replace=False)):
            z = q[n, k]
            step = 7 if i % 3 == 2 else 1
            q[n, k] = z + step if z + step <= 15 else z - step
    scales = g.uniform(0.005, 0.02, size=(N, G)).astype(np.float16).view(np.uint16)
    return {"qweight": _pack_codes(q), "scales": scales, "zeros": zeros, "N": N, "K": K,
            "group": group, "bits": 4}


def outlier_activations(seed: int, T: int, K: int, dtype: str, big: float = 64.0) -> np.ndarray:
    """N(0,1) with one outlier of magnitude `big` in every 128-wide group (its
    position and sign vary by token and group)."""
    g = np.random.default_rng([seed, T, K, 7])
    x = g.standard_normal((T, K), dtype=np.float32)
    for t in range(T):
        for b in range(K // 128):
            x[t, 128 * b + int(g.integers(0, 128))] = np.float32(big if g.integers(0, 2) else -big)
    return workloads.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _linear(w, x, xd, od, flags=0, epi=0):
    import torch
    import ffn_int4_g128_amd as q
    packed = pack_canonical(w, flags)
    xt = bf16_dev(x) if xd == "bf16" else to_dev(x)
    dt = torch.bfloat16 if od == "bf16" else torch.float32
    y = q.qlinear(xt, packed, w["N"], flags=flags, out_dtype=dt, epilogue=epi)
    torch.cuda.synchronize()
    return to_f64(y)


@pytest.mark.parametrize("T,K,xd", [(1, 4096, "bf16"), (5, 4096, "bf16"), (32, 4096, "bf16"),
                                    (17, 13824, "bf16"), (3, 1024, "f32"), (20, 512, "f32")])
def test_one_code_off_zero_point_with_outliers(T, K, xd):
    """Rows with 0, 1, 2 or 5 codes off the zero point; outlier 64 in every
    group.  Row 0 must come out exactly 0."""
    N = 80
    off = [0] + [1 + (n % 3 == 0) + 3 * (n % 7 == 0) for n in range(1, N)]
    w = sparse_weights(11, N, K, off)
    x = outlier_activations(12, T, K, xd)
    got = _linear(w, x, xd, "f32")
    ref, S = oracle.linear(oracle.widen(x, xd), w["qweight"], w["scales"], w["zeros"], N, K)
    assert np.all(ref[:, 0] == 0.0)
    assert_within(got, ref, oracle.C_TOL * S, f"off-zero codes T{T} K{K} {xd}")


@pytest.mark.parametrize("T", [1, 12])
def test_one_code_off_zero_point_silu_mul(T):
    """The fused SiLU(gate)*up epilogue on the same kind of rows (gate and up
    both sparse), against the oracle's first-order tolerance."""
    import ffn_int4_g128_amd as q
    I, K = 48, 4096
    off = [1 + (n % 4) for n in range(2 * I)]
    w = sparse_weights(13, 2 * I, K, off)
    x = outlier_activations(14, T, K, "bf16")
    got = _linear(w, x, "bf16", "f32", flags=q.QI4_PACK_GATEUP, epi=q.QI4_EPI_SILU_MUL)
    h, tol = oracle.gate_up_silu(oracle.widen(x, "bf16"), w["qweight"], w["scales"], w["zeros"],
                                 I, K)
    assert_within(got, h, tol, f"off-zero silu_mul T{T}")


def _sparse_experts(seed, E, H, I):
    ex = {"gu_q": [], "gu_s": [], "gu_z": [], "dn_q": [], "dn_s": [], "dn_z": []}
    for e in range(E + 1):
        gu = sparse_weights(seed + 2 * e, 2 * I, H, [1 + (n % 5) for n in range(2 * I)])
        dn = sparse_weights(seed + 2 * e + 1, H, I, [1 + (n % 3) for n in range(H)])
        for k, d in (("gu", gu), ("dn", dn)):
            ex[k + "_q"].append(d["qweight"])
            ex[k + "_s"].append(d["scales"])
            ex[k + "_z"].append(d["zeros"])
    routed = {k: np.stack(v[:E]) for k, v in ex.items()}
    shared = {k: v[E] for k, v in ex.items()}
    return routed, shared


@pytest.mark.parametrize("T", [5, 40, 200])
def test_moe_sparse_codes_with_outliers(T):
    """A MoE layer whose experts hold mostly zero-point codes, fed activations
    with outliers, on the decode GEMMs (T < 128) and the prefill path."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 1024, 256, 2
    ex, sh = _sparse_experts(15, E, H, I)
    x = outlier_activations(16, T, H, "bf16", big=32.0)
    logits = workloads.logits_normal(17, T, T, E)
    mw = q.pack_moe(ex, sh, E, H, I)
    out = q.moe_ffn(bf16_dev(x), mw, k, logits=to_dev(logits))
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, k)
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E)
    assert_within(to_f64(out), ref, tol, f"moe sparse codes T{T}")


# bf16 bit patterns of +inf and a quiet NaN
_BF16_INF, _BF16_NAN = 0x7F80, 0x7FC0


@pytest.mark.parametrize("T,K,bad", [(3, 4096, _BF16_INF), (20, 4096, _BF16_NAN),
                                     (40, 2048, _BF16_INF)])
def test_nonfinite_row_leaves_other_rows(T, K, bad):
    """One activation row holding an inf or NaN: the header leaves that row's
    outputs unspecified; every other row must still match the oracle (rows
    converted into LDS at T = 3, in registers / row-major beyond 16 rows)."""
    N = 96
    w = workloads.weights(18, T, N, K, 0.005, 0.02)
    x = workloads.activations(19, T, T, K, "bf16").copy()
    r = T // 2
    x[r, 5] = bad
    got = _linear(w, x, "bf16", "f32")
    keep = [t for t in range(T) if t != r]
    ref, S = oracle.linear(oracle.widen(x[keep], "bf16"), w["qweight"], w["scales"], w["zeros"],
                           N, K)
    assert_within(got[keep], ref, oracle.C_TOL * S, f"nonfinite row {r} of T{T}")


@pytest.mark.parametrize("T", [8, 150])
def test_moe_nonfinite_token_leaves_other_tokens(T):
    """The MoE layer with one token's input row holding a NaN: every other
    token matches the oracle (decode GEMMs at T = 8, prefill path at T = 150)."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 512, 256, 2
    ex = workloads.moe_experts(20, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(20, 0, H, I, 0.005, 0.02)
    x = workloads.activations(21, T, T, H, "bf16").copy()
    r = 3
    x[r, 77] = _BF16_NAN
    logits = workloads.logits_normal(22, T, T, E)
    mw = q.pack_moe(ex, sh, E, H, I)
    out = to_f64(q.moe_ffn(bf16_dev(x), mw, k, logits=to_dev(logits)))
    torch.cuda.synchronize()
    keep = [t for t in range(T) if t != r]
    oids, op = oracle.topk_softmax(logits, k)
    ref, tol = oracle.moe(oracle.widen(x[keep], "bf16"), oids[keep], op[keep], ex, sh, H, I, E)
    assert_within(out[keep], ref, tol, f"moe nonfinite token {r} of T{T}")
