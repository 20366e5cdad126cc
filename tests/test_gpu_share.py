"""GPU parity of moe_ffn_int4_share, one device's share of a MoE layer whose
experts are split between devices (the fastllm hybrid placement, read here as
GPU experts plus the rest elsewhere): the share against the oracle with the
other experts' combine weights set to 0; the share plus the oracle's remainder
against the full oracle layer; the routing returned in full; and the other
experts' weight blocks never read (they are filled with NaN scales)."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

E, H, I, K = 16, 512, 256, 4
ON_GPU = [0, 3, 5, 6, 9, 12, 15]


@pytest.fixture(scope="module")
def layer():
    import torch
    import ffn_int4_g128_amd as q
    ex = workloads.moe_experts(140, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(140, 0, H, I, 0.005, 0.02)
    mw = q.pack_moe(ex, sh, E, H, I)
    # the blocks of the experts that run elsewhere: all bytes 0xFF (scales NaN),
    # so any use of them would show in the output
    gu_b = q.packed_bytes(2 * I, H, q.QI4_PACK_GATEUP)
    dn_b = q.packed_bytes(H, I, 0)
    for e in range(E):
        if e not in ON_GPU:
            mw.w_gate_up[e * gu_b:(e + 1) * gu_b].fill_(0xFF)
            mw.w_down[e * dn_b:(e + 1) * dn_b].fill_(0xFF)
    mask = torch.zeros(E, dtype=torch.uint8, device="cuda")
    mask[ON_GPU] = 1
    torch.cuda.synchronize()
    return ex, sh, mw, mask


@pytest.mark.parametrize("T", [1, 5, 40, 150])
def test_share_plus_remainder_is_the_layer(layer, T):
    import torch
    ex, sh, mw, mask = layer
    import ffn_int4_g128_amd as q
    x = workloads.activations(141, T, T, H, "bf16")
    logits = workloads.logits_normal(142, T, T, E)
    out, ids, wts = q.moe_ffn_share(bf16_dev(x), mw, K, mask, logits=to_dev(logits),
                                    return_routing=True)
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, K)
    assert np.array_equal(ids.cpu().numpy(), oids)   # the routing comes back in full
    here = np.isin(oids, ON_GPU)
    x64 = oracle.widen(x, "bf16")
    share, tol_share = oracle.moe(x64, oids, np.where(here, op, 0.0), ex, sh, H, I, E)
    rest, tol_rest = oracle.moe(x64, oids, np.where(here, 0.0, op), ex, None, H, I, E)
    full, tol_full = oracle.moe(x64, oids, op, ex, sh, H, I, E)
    got = to_f64(out)
    assert np.isfinite(got).all()
    assert_within(got, share, tol_share, f"share T{T}")
    assert_within(got + rest, full, tol_full, f"share + remainder T{T}")


def test_all_experts_here_is_moe_ffn_and_none_is_the_shared_expert(layer):
    import torch
    import ffn_int4_g128_amd as q
    ex, sh, _, _ = layer
    T = 12
    mw = q.pack_moe(ex, sh, E, H, I)          # unpoisoned copy
    x = bf16_dev(workloads.activations(143, 0, T, H, "bf16"))
    lg = to_dev(workloads.logits_normal(144, 0, T, E))
    allm = torch.ones(E, dtype=torch.uint8, device="cuda")
    nonem = torch.zeros(E, dtype=torch.uint8, device="cuda")
    a = q.moe_ffn_share(x, mw, K, allm, logits=lg)
    b = q.moe_ffn(x, mw, K, logits=lg)
    c = q.moe_ffn_share(x, mw, K, nonem, logits=lg)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref, tol = oracle.moe(oracle.widen(workloads.activations(143, 0, T, H, "bf16"), "bf16"),
                          np.zeros((T, 1), np.int32), np.zeros((T, 1)), ex, sh, H, I, E)
    assert_within(to_f64(c), ref, tol, "no routed expert here: shared expert only")
