"""Seeded synthetic inputs for the int4-g128 linear and MoE FFN workloads.

This module only draws random inputs and stores them in the canonical
interchange format (the one both the oracle and the GPU library accept).  It
holds none of the method's arithmetic: no dequantization, no products, no
routing.  Both the GPU path and the oracle consume its output.

Canonical format of one quantized matrix W [N][K] (out x in), group size G=128
along K:
  qweight  uint8 [N][K/2]   two 4-bit codes per byte, even k in the low nibble
  scales   uint16 [N][K/G]  IEEE binary16 bit patterns
  zeros    uint8 [N][K/G]   zero point, 0..15
Activations are bf16 bit patterns (uint16) or float32.

Every tensor draws from its own stream ``numpy.random.default_rng([seed, tag...])``.
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# tensor tags (stream ids)
_T_QW, _T_SC, _T_ZR, _T_X, _T_LOGIT, _T_PERM, _T_ROUTER = 1, 2, 3, 4, 5, 6, 7


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs are finite (the generators never draw NaN or infinity)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- weights ------------------------------------------------------------------

def weights(seed: int, tag: int, N: int, K: int, scale_lo: float, scale_hi: float,
            group: int = GROUP, bits: int = 4) -> dict:
    """q uniform in 0..15 (so a packed byte is uniform in 0..255), zero uniform in
    0..15, scale uniform in [scale_lo, scale_hi] rounded to binary16.  group 0 means
    one group per row.  bits 8: q and zero uniform in 0..255, one code per byte
    (qweight [N][K])."""
    group = group or K
    assert K % group == 0 and K % 2 == 0 and bits in (4, 8)
    G = K // group
    qw = rng(seed, tag, _T_QW).integers(0, 256, size=(N, K if bits == 8 else K // 2),
                                        dtype=np.uint8)
    sc = rng(seed, tag, _T_SC).uniform(scale_lo, scale_hi, size=(N, G)).astype(np.float16)
    zr = rng(seed, tag, _T_ZR).integers(0, 1 << bits, size=(N, G), dtype=np.uint8)
    return {"qweight": qw, "scales": sc.view(np.uint16), "zeros": zr, "N": N, "K": K,
            "group": group, "bits": bits}


def activations(seed: int, tag: int, T: int, K: int, dtype: str = "bf16",
                scale: float = 1.0) -> np.ndarray:
    """scale * N(0,1) drawn in float32, then rounded to bf16 (uint16 bits) or kept f32."""
    x = rng(seed, tag, _T_X).standard_normal(size=(T, K), dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


# ---- router logits ---------------------------------------------------------------

def _distinct_rows(draw, T: int, E: int) -> np.ndarray:
    out = np.empty((T, E), dtype=np.float32)
    for t in range(T):
        attempt = 0
        while True:
            row = draw(t, attempt)
            if np.unique(row).size == E:
                break
            attempt += 1
        out[t] = row
    return out


def router_weights(seed: int, tag: int, E: int, H: int) -> np.ndarray:
    """Router matrix [E][H] as bf16 bits: N(0, 1/H) drawn in float32 and rounded,
    so that logits of N(0,1) activations are about N(0,1)."""
    w = rng(seed, tag, _T_ROUTER).standard_normal(size=(E, H), dtype=np.float32)
    w = (w * np.float32(1.0 / np.sqrt(H))).astype(np.float32)
    return f32_to_bf16_bits(w)


def logits_normal(seed: int, tag: int, T: int, E: int) -> np.ndarray:
    """N(0,1) float32 router logits, each row resampled until its values are distinct."""
    return _distinct_rows(
        lambda t, a: rng(seed, tag, _T_LOGIT, t, a).standard_normal(E, dtype=np.float32), T, E)


def zipf_probs(E: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def logits_zipf(seed: int, tag: int, T: int, E: int, s: float = 1.1) -> np.ndarray:
    """Skewed routing: logits[t][e] = ln p_{pi(e)} + Gumbel(0,1), p_r ~ r^-s, pi a
    seeded permutation of the experts.  The top-k of such a row is a draw without
    replacement with probabilities proportional to a Zipf(s) law, so expert loads
    follow a capped Zipf(s) skew.  Rows are resampled until distinct."""
    perm = rng(seed, tag, _T_PERM).permutation(E)
    lp = np.log(zipf_probs(E, s))[perm].astype(np.float32)

    def draw(t, a):
        g = rng(seed, tag, _T_LOGIT, t, a).gumbel(size=E).astype(np.float32)
        return (lp + g).astype(np.float32)
    return _distinct_rows(draw, T, E)


# ---- MoE expert weights ------------------------------------------------------------

def moe_experts(seed: int, layer: int, E: int, H: int, I: int, scale_lo: float,
                scale_hi: float, group: int = GROUP, bits: int = 4) -> dict:
    """Canonical weights of E routed experts stacked on a leading axis:
    gu_* is the [gate; up] matrix (2I x H), dn_* the down matrix (H x I)."""
    gu = [weights(seed, 1000 * layer + 10 * e + 1 + 100000, 2 * I, H, scale_lo, scale_hi, group,
                  bits) for e in range(E)]
    dn = [weights(seed, 1000 * layer + 10 * e + 2 + 100000, H, I, scale_lo, scale_hi, group,
                  bits) for e in range(E)]
    return {"gu_q": np.stack([w["qweight"] for w in gu]),
            "gu_s": np.stack([w["scales"] for w in gu]),
            "gu_z": np.stack([w["zeros"] for w in gu]),
            "dn_q": np.stack([w["qweight"] for w in dn]),
            "dn_s": np.stack([w["scales"] for w in dn]),
            "dn_z": np.stack([w["zeros"] for w in dn])}


def moe_shared(seed: int, layer: int, H: int, I: int, scale_lo: float, scale_hi: float,
               group: int = GROUP, bits: int = 4) -> dict:
    gu = weights(seed, 1000 * layer + 7, 2 * I, H, scale_lo, scale_hi, group, bits)
    dn = weights(seed, 1000 * layer + 8, H, I, scale_lo, scale_hi, group, bits)
    return {"gu_q": gu["qweight"], "gu_s": gu["scales"], "gu_z": gu["zeros"],
            "dn_q": dn["qweight"], "dn_s": dn["scales"], "dn_z": dn["zeros"]}


# ---- the five workloads --------------------------------------------------------

#: one small GEMV, fp32 activations and output
GEMV_SMALL = dict(name="gemv_k256_n128_f32", T=1, K=256, N=128, scale=(0.005, 0.02), seed=0)
#: Llama-7B-shaped decode linear stack (T=1), bf16 in/out
LLAMA7B_STACK = dict(name="llama7b_decode_stack_t1", T=1, seed=1, scale=(0.005, 0.02),
                     linears=[("qkv", 4096, 12288, None), ("o", 4096, 4096, None),
                              ("gate_up", 4096, 2 * 11008, "silu_mul"), ("down", 11008, 4096, None)])
#: skinny decode GEMM sweep
SKINNY_SWEEP = dict(name="skinny_decode_sweep", seed=2, scale=(0.002, 0.01), x_scale=0.5,
                    shapes=[(5120, 13824), (13824, 5120)], T=[1, 4, 8, 16, 32])
#: DeepSeek-V3-shaped MoE expert FFN, decode
MOE_DECODE = dict(name="moe_deepseekv3_shape_decode", seed=3, H=7168, I=2048, E=256, top_k=8,
                  shared=1, scale=(0.005, 0.02), T=[1, 8, 32])
#: the same MoE layer at prefill size with Zipf(1.1)-skewed routing
MOE_PREFILL = dict(name="moe_deepseekv3_shape_prefill", seed=4, H=7168, I=2048, E=256, top_k=8,
                   shared=1, scale=(0.005, 0.02), T=2048, zipf=1.1)


# ---- algorithmic bytes (measurement bookkeeping, not the method) ------------------

def packed_weight_bytes(n_weights: int, group: int = GROUP, bits: int = 4) -> float:
    """Algorithmic bytes of quantized weights: per group of `group` weights,
    group * bits / 8 bytes of codes, a 2-byte binary16 scale and a bits-wide zero
    point."""
    return n_weights * (group * bits / 8 + 2 + bits / 8) / group
