"""GPU parity of the grouped down GEMM in both of its work splits, on one layer:
with enough (expert, quad) pairs (3000 or more: here 129 problems x 32 quads
at T = 32) each wave streams a quad of tiles over the whole K and stores it
from its registers; with fewer (T = 4: 33 problems) the waves split K and
reduce through LDS.  128- and 64-wide groups, 4- and 8-bit codes; every token
against the oracle's MoE layer (the FastLLM page's section 4.2 for the group
sizes; the fastllm README's int4/int8 formats for the code widths)."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

E, H, I, K_TOP = 128, 2048, 128, 8


@pytest.fixture(scope="module", params=[(128, 4), (64, 4), (128, 8)],
                ids=["g128-int4", "g64-int4", "g128-int8"])
def layer(request):
    import torch
    import ffn_int4_g128_amd as q
    group, bits = request.param
    ex = workloads.moe_experts(150, bits, E, H, I, 0.005, 0.02, group=group, bits=bits)
    sh = workloads.moe_shared(150, bits, H, I, 0.005, 0.02, group=group, bits=bits)
    mw = q.pack_moe(ex, sh, E, H, I, group=group, flags=q.QI4_INT8 if bits == 8 else 0)
    torch.cuda.synchronize()
    yield group, bits, ex, sh, mw
    del mw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [4, 32])
def test_down_work_splits(layer, T):
    import torch
    import ffn_int4_g128_amd as q
    group, bits, ex, sh, mw = layer
    print(f"[down splits] group {group} bits {bits} T={T} launching", flush=True)
    x = workloads.activations(151, T, T, H, "bf16")
    logits = workloads.logits_normal(152, T, T, E)
    out, ids, wts = q.moe_ffn(bf16_dev(x), mw, K_TOP, logits=to_dev(logits), return_routing=True)
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, K_TOP)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E, group=group,
                          bits=bits)
    got = to_f64(out)
    assert np.isfinite(got).all()
    assert_within(got, ref, tol, f"group {group} bits {bits} T{T}")
