"""GPU parity of the MoE path against the oracle: router ids and the token
permutation bit for bit, combine weights, the stage calls, and moe_ffn_int4 on
small layers and on the DeepSeek-V3-shaped layer (decode T in {1, 8, 32}, every
token, and the Zipf-skewed prefill T = 2048, a block of 128 tokens that reaches
every tile class).  Output
tolerance: the oracle's first-order composite bound (per-linear factor 2e-3
propagated through SiLU(g)*u, the down projection and the combine)."""
import numpy as np
import pytest

import oracle
import workloads
from tests._gpu import assert_within, bf16_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (8, 256, 8), (32, 256, 8), (2048, 256, 8),
                                   (5, 16, 3), (70, 64, 1), (3, 1000, 32), (9, 8, 8)])
def test_route_topk_bit_exact(T, E, k):
    import ffn_int4_g128_amd as q
    logits = workloads.logits_normal(61, E + k, T, E)
    ids, wts = q.moe_route_topk(to_dev(logits), k)
    oids, op = oracle.topk_softmax(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(wts.cpu().numpy().astype(np.float64) - op)) <= oracle.EPS_P


def test_route_topk_ties_go_to_lower_index():
    import ffn_int4_g128_amd as q
    g = np.random.default_rng(0)
    logits = g.integers(-2, 3, size=(40, 64)).astype(np.float32)
    logits[0] = 0.0
    ids, _ = q.moe_route_topk(to_dev(logits), 8)
    oids, _ = oracle.topk_softmax(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), oids)


def test_route_zipf_prefill_bit_exact():
    import ffn_int4_g128_amd as q
    c = workloads.MOE_PREFILL
    logits = workloads.logits_zipf(c["seed"], 5, c["T"], c["E"], c["zipf"])
    ids, wts = q.moe_route_topk(to_dev(logits), c["top_k"])
    oids, op = oracle.topk_softmax(logits, c["top_k"])
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(wts.cpu().numpy().astype(np.float64) - op)) <= oracle.EPS_P


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (32, 256, 8), (2048, 256, 8), (7, 16, 4),
                                   (300, 1024, 8), (1, 1, 1), (100, 8, 8)])
def test_sort_tokens_bit_exact(T, E, k):
    import ffn_int4_g128_amd as q
    if E == 1:
        ids = np.zeros((T, k), dtype=np.int32)
    else:
        ids, _ = oracle.topk_softmax(workloads.logits_normal(62, T, T, E), k)
    sp, off, inv, act = q.moe_sort_tokens(to_dev(ids), E)
    osp, ooff, oinv = oracle.sort_tokens(ids, E)
    assert np.array_equal(sp.cpu().numpy(), osp)
    assert np.array_equal(off.cpu().numpy(), ooff)
    assert np.array_equal(inv.cpu().numpy(), oinv)
    a = act.cpu().numpy()
    nonempty = np.nonzero(np.diff(ooff))[0]
    assert a[0] == len(nonempty) and np.array_equal(a[1:1 + a[0]], nonempty)


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (4, 256, 8), (5, 256, 8), (4, 1024, 32),
                                   (8, 256, 8), (16, 256, 8), (17, 256, 8),
                                   (32, 256, 8), (2048, 256, 8), (3, 1000, 32), (9, 8, 8),
                                   (16, 1024, 32), (17, 1024, 32), (70, 64, 1), (1, 1, 1)])
def test_route_sort_bit_exact(T, E, k):
    """The routing + permutation call (one fused workgroup of 4 waves up to 4
    tokens, of 16 up to 16 tokens, else the two kernels) gives the oracle's ids
    and permutation bit for bit."""
    import ffn_int4_g128_amd as q
    logits = workloads.logits_normal(63, E + k, T, E)
    ids, wts, sp, off, inv, act = q.moe_route_sort(to_dev(logits), k)
    oids, op = oracle.topk_softmax(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(wts.cpu().numpy().astype(np.float64) - op)) <= oracle.EPS_P
    osp, ooff, oinv = oracle.sort_tokens(oids, E)
    assert np.array_equal(sp.cpu().numpy(), osp)
    assert np.array_equal(off.cpu().numpy(), ooff)
    assert np.array_equal(inv.cpu().numpy(), oinv)
    a = act.cpu().numpy()
    nonempty = np.nonzero(np.diff(ooff))[0]
    assert a[0] == len(nonempty) and np.array_equal(a[1:1 + a[0]], nonempty)


def _small_layer(E, H, I, seed, shared=True):
    ex = workloads.moe_experts(seed, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(seed, 0, H, I, 0.005, 0.02) if shared else None
    return ex, sh


@pytest.mark.parametrize("T,E,H,I,k,shared", [(1, 8, 256, 128, 2, True), (5, 8, 256, 128, 2, True),
                                              (33, 16, 384, 256, 4, True), (17, 6, 128, 128, 6, False),
                                              (64, 4, 256, 128, 1, True), (127, 8, 256, 128, 2, True),
                                              (128, 8, 256, 128, 2, True), (300, 16, 384, 256, 4, True),
                                              (200, 6, 128, 384, 6, False), (513, 32, 512, 128, 8, True),
                                              # the shared expert's problems per decode launch change
                                              # at 8 / 9 tokens (down, 8-slot M tiles) and at 16 / 17
                                              # (gate/up, 16 slots)
                                              (8, 8, 256, 128, 2, True), (9, 8, 256, 128, 2, True),
                                              (16, 8, 256, 128, 2, True), (17, 8, 256, 128, 2, True)])
def test_moe_small_layers(T, E, H, I, k, shared):
    import torch
    import ffn_int4_g128_amd as q
    ex, sh = _small_layer(E, H, I, 70 + T, shared)
    x = workloads.activations(71, T, T, H, "bf16")
    logits = workloads.logits_normal(72, T, T, E)
    mw = q.pack_moe(ex, sh, E, H, I)
    out, ids, wts = q.moe_ffn(bf16_dev(x), mw, k, logits=to_dev(logits), return_routing=True)
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E)
    assert_within(to_f64(out), ref, tol, f"moe T{T} E{E} H{H} I{I} k{k} shared={shared}")


@pytest.mark.parametrize("T", [12, 150])
def test_moe_given_routing_and_stage_calls_agree(T):
    """Passing ids/weights instead of logits, and running the five stages by hand,
    give the same bits as the one-call path (decode and prefill sizes)."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 256, 128, 3
    ex, sh = _small_layer(E, H, I, 80)
    x = bf16_dev(workloads.activations(81, 0, T, H, "bf16"))
    lg = to_dev(workloads.logits_normal(82, 0, T, E))
    mw = q.pack_moe(ex, sh, E, H, I)
    a, ids, wts = q.moe_ffn(x, mw, k, logits=lg, return_routing=True)
    b = q.moe_ffn(x, mw, k, ids=ids, weights=wts)
    sp, off, inv, act = q.moe_sort_tokens(ids, E)
    h = q.moe_gate_up(x, mw, k, sp, off, act)
    y = q.moe_down(h, T, mw, k, off, act)
    c = q.moe_combine(y, wts, inv, T, mw, k)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_moe_top1_equals_single_expert_linear_path():
    """top-1 routing with weight 1 and no shared expert is one expert's FFN: compare
    with qlinear(SiLU_MUL) followed by qlinear(down) (both already oracle-checked)."""
    import torch
    import ffn_int4_g128_amd as q
    T, E, H, I = 6, 4, 256, 128
    ex, _ = _small_layer(E, H, I, 90, shared=False)
    x = bf16_dev(workloads.activations(91, 0, T, H, "bf16"))
    ids = torch.full((T, 1), 2, dtype=torch.int32, device="cuda")
    wts = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    mw = q.pack_moe(ex, None, E, H, I)
    out = q.moe_ffn(x, mw, 1, ids=ids, weights=wts)
    gu = q.pack(to_dev(ex["gu_q"][2]), to_dev(ex["gu_s"][2]), to_dev(ex["gu_z"][2]), 2 * I, H,
                q.QI4_PACK_GATEUP)
    dn = q.pack(to_dev(ex["dn_q"][2]), to_dev(ex["dn_s"][2]), to_dev(ex["dn_z"][2]), H, I)
    h = q.qlinear(x, gu, 2 * I, flags=q.QI4_PACK_GATEUP, out_dtype=torch.float32,
                  epilogue=q.QI4_EPI_SILU_MUL)
    y = q.qlinear(h, dn, H, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, tol = oracle.moe(oracle.widen(workloads.activations(91, 0, T, H, "bf16"), "bf16"),
                          np.full((T, 1), 2, np.int32), np.ones((T, 1)), ex, None, H, I, E)
    assert_within(to_f64(out), ref, tol, "top-1 moe vs oracle")
    assert_within(to_f64(y), ref, tol, "qlinear chain vs oracle")


@pytest.mark.parametrize("T", [12, 300])
def test_moe_large_scales(T):
    """Scales at and above 256 (where 16 (q - zero) scale leaves binary16) in a
    gate/up row block of one expert and a down row block of another, plus one
    scale just below: the prefill path hands the affected tiles to its
    plain-operand pass; decode sizes take the f32-scale path.  Checked against
    the oracle like any other layer."""
    import torch
    import ffn_int4_g128_amd as q
    E, H, I, k = 8, 384, 256, 4
    ex, sh = _small_layer(E, H, I, 95)
    f16 = lambda v: np.array([v], np.float16).view(np.uint16)[0]
    ex["gu_s"][2, 40:48, 1] = f16(300.0)     # gate rows of expert 2
    ex["gu_s"][2, 300, 2] = f16(256.0)       # up row of expert 2
    ex["dn_s"][5, 100:116, 0] = f16(1000.0)  # down rows of expert 5
    ex["dn_s"][6, 7, 1] = f16(255.9)         # just below: stays on the fast operands
    x = workloads.activations(96, T, T, H, "bf16")
    logits = workloads.logits_normal(97, T, T, E)
    mw = q.pack_moe(ex, sh, E, H, I)
    out = q.moe_ffn(bf16_dev(x), mw, k, logits=to_dev(logits))
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, k)
    assert {2, 5, 6} <= set(np.unique(oids).tolist())
    ref, tol = oracle.moe(oracle.widen(x, "bf16"), oids, op, ex, sh, H, I, E)
    assert np.isfinite(ref).all()
    assert_within(to_f64(out), ref, tol, f"moe large scales T{T}")


# ---- the DeepSeek-V3-shaped layer ----------------------------------------------------

@pytest.fixture(scope="module")
def dsv3():
    import torch
    import ffn_int4_g128_amd as q
    c = workloads.MOE_DECODE
    ex = workloads.moe_experts(c["seed"], 0, c["E"], c["H"], c["I"], *c["scale"])
    sh = workloads.moe_shared(c["seed"], 0, c["H"], c["I"], *c["scale"])
    mw = q.pack_moe(ex, sh, c["E"], c["H"], c["I"])
    torch.cuda.synchronize()
    yield c, ex, sh, mw
    del mw
    torch.cuda.empty_cache()


def _check_layer(c, ex, sh, mw, T, logits, x, tag, sample):
    import torch
    import ffn_int4_g128_amd as q
    print(f"[{tag}] T={T} launching", flush=True)
    out, ids, wts = q.moe_ffn(bf16_dev(x), mw, c["top_k"], logits=to_dev(logits),
                              return_routing=True)
    torch.cuda.synchronize()
    oids, op = oracle.topk_softmax(logits, c["top_k"])
    assert np.array_equal(ids.cpu().numpy(), oids)
    rows = sample
    ref, tol = oracle.moe(oracle.widen(x[rows], "bf16"), oids[rows], op[rows], ex, sh,
                          c["H"], c["I"], c["E"])
    assert_within(to_f64(out)[rows], ref, tol, f"{tag} T{T} tokens {rows}")


@pytest.mark.parametrize("T", workloads.MOE_DECODE["T"])
def test_dsv3_decode(dsv3, T):
    """Every token of the decode batch against the oracle."""
    c, ex, sh, mw = dsv3
    logits = workloads.logits_normal(c["seed"], 10 + T, T, c["E"])
    x = workloads.activations(c["seed"], 20 + T, T, c["H"], "bf16")
    _check_layer(c, ex, sh, mw, T, logits, x, "dsv3 decode", list(range(T)))


def _prefill_tile_classes(ids, E, tokens, big=128, small_max=64):
    """Tile class of each (token, slot) in the prefill planner's cut of each
    expert's rows: 'big' for rows in a 65..128-row tile, else the small-tile
    class of its expert's remainder (<=16, <=32, <=64 rows).  Computed from the
    oracle's permutation: a pair's row within its expert's segment and the
    segment's length."""
    sp, off, _ = oracle.sort_tokens(ids, E)
    k = ids.shape[1]
    pos = np.empty(ids.size, dtype=np.int64)
    pos[sp] = np.arange(ids.size)
    classes = set()
    for t in tokens:
        for j in range(k):
            e = ids[t, j]
            n = off[e + 1] - off[e]
            r = pos[t * k + j] - off[e]
            full, rem = n // big, n % big
            if r < full * big or rem > small_max:
                classes.add("big")
            else:
                classes.add("le16" if rem <= 16 else "le32" if rem <= 32 else "le64")
    return classes


def test_dsv3_prefill_zipf(dsv3):
    """The Zipf-skewed T=2048 prefill: 128 consecutive tokens (the last ones, in
    the shared expert's last tile) plus the first, against the oracle.  The
    block reaches rows in big tiles and in small tiles of every height class."""
    c, ex, sh, mw = dsv3
    p = workloads.MOE_PREFILL
    T = p["T"]
    logits = workloads.logits_zipf(p["seed"], 5, T, p["E"], p["zipf"])
    x = workloads.activations(p["seed"], 6, T, p["H"], "bf16")
    tokens = [0] + list(range(T - 128, T))
    oids, _ = oracle.topk_softmax(logits, p["top_k"])
    assert _prefill_tile_classes(oids, p["E"], tokens) == {"big", "le16", "le32", "le64"}
    _check_layer(c, ex, sh, mw, T, logits, x, "dsv3 prefill zipf", tokens)


@pytest.mark.parametrize("T", [32, 2048])
def test_dsv3_layer_is_deterministic(dsv3, T):
    """Two calls on the same inputs give bit-identical outputs on the decode path
    and on the prefill path (every output element is reduced in a fixed order)."""
    import torch
    import ffn_int4_g128_amd as q
    c, ex, sh, mw = dsv3
    logits = to_dev(workloads.logits_zipf(4, 9, T, c["E"], 1.1))
    x = bf16_dev(workloads.activations(4, 8, T, c["H"], "bf16"))
    a = q.moe_ffn(x, mw, c["top_k"], logits=logits)
    b = q.moe_ffn(x, mw, c["top_k"], logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,E,H,k", [(1, 256, 7168, 8), (32, 256, 7168, 8), (5, 64, 512, 4),
                                     (70, 300, 1024, 8), (2048, 256, 7168, 8), (3, 8, 32, 8),
                                     # the decode path's last token count and the first past it
                                     (64, 256, 1024, 8), (65, 256, 1024, 8), (2, 17, 96, 3)])
def test_router_logits_and_topk(T, E, H, k):
    """Router projection within 2e-3 * sum|x*w| of the oracle; the selection on the
    GPU's logits bit for bit (the same decision in the same precision), and valid
    against the oracle's logits within that tolerance."""
    import torch
    import ffn_int4_g128_amd as q
    w = workloads.router_weights(88, E + H, E, H)
    x = workloads.activations(89, T, T, H, "bf16")
    logits, ids, wts = q.moe_router_topk(bf16_dev(x), bf16_dev(w), k)
    torch.cuda.synchronize()
    L, S = oracle.router_logits(oracle.widen(x, "bf16"), w)
    got = logits.cpu().numpy()
    tol = oracle.C_TOL * S
    assert_within(got.astype(np.float64), L, tol, f"router T{T} E{E} H{H}")
    oids, op = oracle.topk_softmax(got, k)
    gids = ids.cpu().numpy()
    assert np.array_equal(gids, oids)
    assert np.max(np.abs(wts.cpu().numpy().astype(np.float64) - op)) <= oracle.EPS_P
    # every selected expert is within tolerance of every one left out
    for t in range(T):
        sel = np.zeros(E, dtype=bool)
        sel[gids[t]] = True
        if sel.all():
            continue
        assert np.min(L[t, sel] + tol[t, sel]) >= np.max(L[t, ~sel] - tol[t, ~sel])
