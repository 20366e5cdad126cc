"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on the
caller's stream): every replay, with eager work and synchronizations between
the replays, must give bit for bit the eager call's output.  Covers the dense
linear with one row (rows converted into LDS) and with 40 rows (rows split over
grid.y, loaded row-major), and the MoE layer on its decode path (T = 8) and its
prefill path (T = 160: plan, big and small tiles, deferred list)."""
import pytest

import workloads
from tests._gpu import bf16_dev, pack_canonical, to_dev

pytestmark = pytest.mark.gpu


def _replays_match(capture_fn, out, eager, what):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_fn()
    for r in range(3):
        out.fill_(float("nan"))        # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"{what}: replay {r} differs from the eager call"
    del g


@pytest.mark.parametrize("T", [1, 40])
def test_qlinear_graph_replays(T):
    import torch
    import ffn_int4_g128_amd as q
    N, K = 1000, 4096
    w = workloads.weights(71, T, N, K, 0.005, 0.02)
    x = bf16_dev(workloads.activations(71, T + 1, T, K, "bf16"))
    packed = pack_canonical(w)
    print(f"[graph] qlinear T={T} N={N} K={K}", flush=True)
    eager = q.qlinear(x, packed, N, out_dtype=torch.float32).clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    _replays_match(lambda: q.qlinear(x, packed, N, out=out), out, eager, f"qlinear T{T}")


@pytest.mark.parametrize("T", [8, 160])
def test_moe_graph_replays(T):
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 16, 512, 256, 4
    ex = workloads.moe_experts(72, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(72, 0, H, I, 0.005, 0.02)
    mw = q.pack_moe(ex, sh, E, H, I)
    x = bf16_dev(workloads.activations(73, T, T, H, "bf16"))
    logits = to_dev(workloads.logits_normal(74, T, T, E))
    print(f"[graph] moe_ffn T={T} E={E} H={H} I={I} k={k}", flush=True)
    eager = q.moe_ffn(x, mw, k, logits=logits).clone()
    ws = q.moe_workspace(mw, k, T, x.device)
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    _replays_match(lambda: q.moe_ffn(x, mw, k, logits=logits, workspace=ws, out=out), out, eager,
                   f"moe T{T}")
