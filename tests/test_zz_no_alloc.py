"""moe_ffn_int4_noalloc, the MoE layer for callers that cannot allocate: called
through the C ABI, it must give moe_ffn_int4's outputs bit for bit (same
kernels, the library's per-GPU scratch array in place of the caller's
workspace), on consecutive calls whose second input is smaller than the first
(the array keeps the previous call's contents), on the decode and the prefill
paths, and it must reject a layer too large for the array before launching
anything.  Captured in a HIP graph, its replays give the eager output."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _layer(E, H, I, seed):
    import ffn_int4_g128_amd as q
    ex = workloads.moe_experts(seed, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(seed, 0, H, I, 0.005, 0.02)
    return ex, sh, q.pack_moe(ex, sh, E, H, I)


@pytest.mark.parametrize("Ts", [(40, 7), (200, 130, 3)])
def test_noalloc_matches_workspace_call_bit_for_bit(Ts):
    """Consecutive calls, each smaller than the one before: decode sizes, then
    the prefill path (T >= 128) followed by smaller batches."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 512, 256, 2
    ex, sh, mw = _layer(E, H, I, 120)
    for i, T in enumerate(Ts):
        x = workloads.activations(121, 10 * i + T, T, H, "bf16")
        logits = workloads.logits_normal(122, 10 * i + T, T, E)
        xt, lt = bf16_dev(x), to_dev(logits)
        print(f"noalloc call {i}: T={T}", flush=True)
        got, ids, wts = q.moe_ffn_noalloc(xt, mw, k, logits=lt, return_routing=True)
        ref, rids, rwts = q.moe_ffn(xt, mw, k, logits=lt, return_routing=True)
        torch.cuda.synchronize()
        assert torch.equal(ids, rids) and torch.equal(wts, rwts)
        assert torch.equal(got, ref), f"call {i} (T={T}) differs from moe_ffn_int4"
        oids, op = oracle.topk_softmax(logits, k)
        o, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E)
        assert_within(to_f64(got), o, tol, f"noalloc T{T}")


def test_noalloc_given_routing_and_dsv3_shape_limit():
    """Routing passed in (ids and weights) instead of logits; and the
    DeepSeek-V3 shape at T = 256 needs more scratch than the array holds: the
    call returns QI4_ERR_WORKSPACE without touching anything."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k, T = 8, 256, 128, 3, 9
    ex, sh, mw = _layer(E, H, I, 130)
    xt = bf16_dev(workloads.activations(131, 0, T, H, "bf16"))
    ids, wts = q.moe_route_topk(to_dev(workloads.logits_normal(132, 0, T, E)), k)
    got = q.moe_ffn_noalloc(xt, mw, k, ids=ids, weights=wts)
    ref = q.moe_ffn(xt, mw, k, ids=ids, weights=wts)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)

    d = q._MoeDesc(256, 7168, 2048, 8, 128, 1, 0)
    need = q.lib().moe_ffn_int4_workspace_bytes(ctypes.byref(d), 256)
    assert need > q.NOALLOC_SCRATCH_BYTES
    assert q.lib().moe_ffn_int4_workspace_bytes(ctypes.byref(d), 128) <= q.NOALLOC_SCRATCH_BYTES
    out = torch.full((256, 7168), 7.0, dtype=torch.bfloat16, device="cuda")
    rc = q.lib().moe_ffn_int4_noalloc(ctypes.byref(d), None, 256, None, None, None, None, None,
                                      None, None, q._ptr(out), q._stream())
    torch.cuda.synchronize()
    assert rc == -5  # QI4_ERR_WORKSPACE
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("T", [8, 150])
def test_noalloc_under_graph_capture(T):
    """The use the entry point is for: captured in a HIP graph (no allocation
    inside the call), every replay, with eager work between, gives the eager
    call's output bit for bit; decode and prefill paths."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 512, 256, 2
    _, _, mw = _layer(E, H, I, 140)
    xt = bf16_dev(workloads.activations(141, T, T, H, "bf16"))
    lt = to_dev(workloads.logits_normal(142, T, T, E))
    print(f"noalloc graph capture: T={T}", flush=True)
    eager = q.moe_ffn_noalloc(xt, mw, k, logits=lt).clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.moe_ffn_noalloc(xt, mw, k, logits=lt, out=out)
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
    del g
