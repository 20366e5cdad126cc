"""Pins of the oracle's router (top-k + softmax), token permutation, MoE FFN and
reference quantizer: brute force, closed forms, library routines, invariants, and
the reduction of top-1 routing to a single expert FFN."""
import math

import numpy as np
import pytest

import oracle
import workloads


# ---- top-k ------------------------------------------------------------------

def _brute_topk(row, k):
    return [i for _, i in sorted((-float(v), i) for i, v in enumerate(row))][:k]


@pytest.mark.parametrize("T,E,k", [(4, 16, 3), (3, 8, 8), (5, 256, 8), (2, 9, 1)])
def test_topk_matches_brute_force(T, E, k):
    logits = workloads.logits_normal(1, E, T, E)
    ids, p = oracle.topk_softmax(logits, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(logits[t], k)


def test_topk_matches_numpy_lexsort_with_ties():
    g = np.random.default_rng(0)
    logits = g.integers(-3, 4, size=(50, 32)).astype(np.float32)  # many ties
    ids, _ = oracle.topk_softmax(logits, 8)
    for t in range(50):
        order = np.lexsort((np.arange(32), -logits[t].astype(np.float64)))
        assert ids[t].tolist() == order[:8].tolist()


def test_topk_special_cases():
    ids, p = oracle.topk_softmax(np.arange(16, dtype=np.float32).reshape(1, 16), 4)
    assert ids[0].tolist() == [15, 14, 13, 12]
    ids, p = oracle.topk_softmax(np.zeros((1, 10), dtype=np.float32), 4)
    assert ids[0].tolist() == [0, 1, 2, 3] and np.all(p == 0.25)


def test_softmax_over_selected():
    from scipy.special import softmax
    logits = workloads.logits_normal(2, 0, 20, 256)
    ids, p = oracle.topk_softmax(logits, 8)
    for t in range(20):
        sel = logits[t, ids[t]].astype(np.float64)
        assert np.allclose(p[t], softmax(sel), rtol=1e-14, atol=0)
        assert abs(p[t].sum() - 1.0) < 1e-15
        assert np.all(np.diff(p[t]) <= 0)  # descending logits give descending weights
    # k = 2 closed form: p0 = 1 / (1 + e^(l1 - l0))
    ids, p = oracle.topk_softmax(np.array([[0.5, 2.0, -1.0]], dtype=np.float32), 2)
    assert p[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(0.5 - 2.0)), rel=1e-15)
    # top-1 gives exactly 1
    _, p1 = oracle.topk_softmax(logits, 1)
    assert np.all(p1 == 1.0)


# ---- permutation ---------------------------------------------------------------

def _check_perm(ids, E, sp, off, inv):
    T, k = ids.shape
    flat = ids.reshape(-1)
    assert off[0] == 0 and off[E] == T * k
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert sorted(sp.tolist()) == list(range(T * k))
    assert np.array_equal(inv[sp], np.arange(T * k))
    for e in range(E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)  # tokens ascending, each token once


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (7, 16, 4), (33, 64, 8), (200, 8, 2)])
def test_sort_invariants_and_brute_force(T, E, k):
    logits = workloads.logits_normal(3, T, T, E)
    ids, _ = oracle.topk_softmax(logits, k)
    sp, off, inv = oracle.sort_tokens(ids, E)
    _check_perm(ids, E, sp, off, inv)
    brute = sorted(range(T * k), key=lambda pr: (int(ids.reshape(-1)[pr]), pr))
    assert sp.tolist() == brute


def test_sort_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.sort_tokens(np.array([[0, 9]], dtype=np.int32), 8)


# ---- MoE ------------------------------------------------------------------------

H, I, E, G = 256, 128, 6, 128


@pytest.fixture(scope="module")
def small_moe():
    ex = workloads.moe_experts(5, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(5, 0, H, I, 0.005, 0.02)
    x = oracle.widen(workloads.activations(5, 1, 4, H, "bf16"), "bf16")
    return ex, sh, x


def _expert(d, e=None):
    pick = (lambda a: a[e]) if e is not None else (lambda a: a)
    return {k: pick(v) for k, v in d.items()}


def test_top1_reduces_to_a_single_expert_ffn(small_moe):
    ex, _, x = small_moe
    T = x.shape[0]
    for e in range(E):
        ids = np.full((T, 1), e, dtype=np.int32)
        p = np.ones((T, 1))
        out, tol = oracle.moe(x, ids, p, ex, None, H, I, E)
        d = _expert(ex, e)
        # the same FFN from independent pieces: numpy matmuls of a numpy dequant
        def deq(qw, s, z, N, K):
            q = np.empty((N, K), dtype=np.int64)
            q[:, 0::2], q[:, 1::2] = qw & 15, qw >> 4
            return (np.repeat(s.view(np.float16).astype(np.float64), G, 1)
                    * (q - np.repeat(z.astype(np.int64), G, 1)))
        Wgu = deq(d["gu_q"], d["gu_s"], d["gu_z"], 2 * I, H)
        Wd = deq(d["dn_q"], d["dn_s"], d["dn_z"], H, I)
        gu = x @ Wgu.T
        g, u = gu[:, :I], gu[:, I:]
        from scipy.special import expit
        ref = (g * expit(g) * u) @ Wd.T
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())
        assert np.all(tol > 0)


def test_identical_experts_sum_to_one_expert_plus_shared(small_moe):
    ex, sh, x = small_moe
    T = x.shape[0]
    same = {k: np.stack([v[2]] * E) for k, v in ex.items()}
    logits = workloads.logits_normal(6, 0, T, E)
    ids, p = oracle.topk_softmax(logits, 4)
    out, _ = oracle.moe(x, ids, p, same, sh, H, I, E)
    one, _ = oracle.moe(x, np.zeros((T, 1), np.int32), np.ones((T, 1)), same, None, H, I, E)
    shared_only, _ = oracle.moe(x, np.zeros((T, 1), np.int32), np.zeros((T, 1)), same, sh, H, I, E)
    assert np.allclose(out, one + shared_only, rtol=1e-12, atol=1e-12 * np.abs(out).max())


def test_zero_combine_weights_leave_only_the_shared_expert(small_moe):
    ex, sh, x = small_moe
    T = x.shape[0]
    ids = np.tile(np.arange(4, dtype=np.int32), (T, 1))
    out, _ = oracle.moe(x, ids, np.zeros((T, 4)), ex, sh, H, I, E)
    shd = {k: v[None] for k, v in sh.items()}
    ref, _ = oracle.moe(x, np.zeros((T, 1), np.int32), np.ones((T, 1)), shd, None, H, I, 1)
    assert np.array_equal(out, ref)


def test_slot_order_does_not_matter(small_moe):
    ex, sh, x = small_moe
    T = x.shape[0]
    ids, p = oracle.topk_softmax(workloads.logits_normal(7, 0, T, E), 3)
    out, tol = oracle.moe(x, ids, p, ex, sh, H, I, E)
    out2, tol2 = oracle.moe(x, ids[:, ::-1].copy(), p[:, ::-1].copy(), ex, sh, H, I, E)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-13 * np.abs(out).max())
    assert np.allclose(tol, tol2, rtol=1e-13)


def test_moe_is_linear_in_combine_weights(small_moe):
    ex, _, x = small_moe
    T = x.shape[0]
    ids = np.tile(np.array([1, 4], dtype=np.int32), (T, 1))
    a, _ = oracle.moe(x, ids, np.tile([1.0, 0.0], (T, 1)), ex, None, H, I, E)
    b, _ = oracle.moe(x, ids, np.tile([0.0, 1.0], (T, 1)), ex, None, H, I, E)
    c, _ = oracle.moe(x, ids, np.tile([0.25, 0.75], (T, 1)), ex, None, H, I, E)
    assert np.allclose(c, 0.25 * a + 0.75 * b, rtol=1e-13, atol=1e-13 * np.abs(c).max())


def test_moe_per_row_groups_match_whole_row_groups_when_hidden_equals_inter():
    # group 0 means one group per row of each matrix; with H == I that is G = H
    Hs = Is = 256
    ex = workloads.moe_experts(41, 0, 4, Hs, Is, 0.005, 0.02, group=0)
    sh = workloads.moe_shared(41, 0, Hs, Is, 0.005, 0.02, group=0)
    x = oracle.widen(workloads.activations(41, 1, 3, Hs, "bf16"), "bf16")
    ids = np.array([[0, 2], [1, 3], [3, 0]], dtype=np.int32)
    p = np.array([[0.6, 0.4], [0.5, 0.5], [0.9, 0.1]])
    a, ta = oracle.moe(x, ids, p, ex, sh, Hs, Is, 4, group=0)
    b, tb = oracle.moe(x, ids, p, ex, sh, Hs, Is, 4, group=Hs)
    assert np.array_equal(a, b) and np.array_equal(ta, tb)


# ---- reference quantizer -----------------------------------------------------------

@pytest.mark.parametrize("G", [128, 64, 256, 512])
def test_quantizer_error_bound_and_dequant_round_trip(G):
    g = np.random.default_rng(9)
    w = g.standard_normal((8, 512)) * 0.05
    w[0, :G] = 0.0          # an all-zero group
    w[1, :G] = 0.37         # a constant positive group (0 joins the range)
    w[2, :G] = -np.abs(w[2, :G])  # an all-negative group
    qw, s, z = oracle.quantize(w, G)
    wd = oracle.dequant(qw, s, z, 8, 512, G)
    sc = np.repeat(s.view(np.float16).astype(np.float64), G, axis=1)
    assert np.all(np.abs(w - wd) <= sc * (0.5 + 1e-3) + 1e-12)
    assert np.all(wd[0, :G] == 0.0)
    # re-quantizing the dequantized grid with its own scale and zero reproduces the codes
    q = oracle.unpack(qw, 8, 512).astype(np.int64)
    zz = np.repeat(z.astype(np.int64), G, axis=1)
    assert np.array_equal(np.clip(np.rint(wd / sc) + zz, 0, 15), q)


# ---- router logits ---------------------------------------------------------------

def test_router_logits_against_exact_rationals():
    from fractions import Fraction
    T, E, H = 3, 5, 64
    w = workloads.router_weights(43, 1, E, H)
    x = oracle.widen(workloads.activations(43, 2, T, H, "bf16"), "bf16")
    y, S = oracle.router_logits(x, w)
    wf = oracle.widen(w, "bf16")
    for t in range(T):
        for e in range(E):
            ex = sum(Fraction(float(x[t, k])) * Fraction(float(wf[e, k])) for k in range(H))
            mag = sum(abs(Fraction(float(x[t, k])) * Fraction(float(wf[e, k]))) for k in range(H))
            assert abs(Fraction(float(y[t, e])) - ex) <= Fraction(2 * H) * Fraction(2.0 ** -53) * mag
            assert abs(Fraction(float(S[t, e])) - mag) <= Fraction(2 * H) * Fraction(2.0 ** -53) * mag


def test_router_logits_one_hot_token_reads_one_weight_column():
    # x = unit vector at k: the logits are column k of the router matrix (rows are
    # experts), which catches a transposed operand
    E, H = 7, 256
    w = workloads.router_weights(44, 1, E, H)
    x = np.zeros((2, H))
    x[0, 3] = 1.0
    x[1, 200] = -2.0
    y, S = oracle.router_logits(x, w)
    wf = oracle.widen(w, "bf16")
    assert np.array_equal(y[0], wf[:, 3]) and np.array_equal(y[1], -2.0 * wf[:, 200])
    assert np.array_equal(S[1], 2.0 * np.abs(wf[:, 200]))
