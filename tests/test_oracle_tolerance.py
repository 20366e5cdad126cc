"""Pins of the oracle's composite tolerances from above and below.

Every GPU parity verdict on a composite (SiLU(gate)*up, the MoE layer, the
W4A8 MoE layer) accepts on a tolerance the oracle computes.  The tolerance is
the first-order worst case of a per-linear error c * sum|w*x| carried through
the composite (reading R14; R30 for W4A8).  These tests check it against what
that definition means, with no use of the oracle's formula: perturb every
linear's result by +-c * sum|w*x| (and the combine weights by +-eps_p), with
the signs that push one output element up the most, evaluate the composite
again in numpy, and require the change to equal the oracle's tolerance.  At a
tiny c the first order is exact to ~1e-5 (second-order terms near
g = 0, where SiLU(g) is small, are the largest), so a dropped or doubled term, a wrong
magnitude (gate for up), or a missing derivative factor moves the ratio away
from 1.  The bound holds beyond first order (the largest SiLU deviation over the
whole interval, the cross terms): at the workloads' c = 2e-3 the ratio stays
within [0.5, 1].

The W4A8 term for int8 decisions of h that could go either way is pinned the
same way: flipping each such decision to its other code changes the output by
exactly one quantization step times |W_d| each, and those add up to the term.

Also here: a hand-computed group for the reference quantizer (binary16 scale
bits, zero point and codes), which a divisor other than 15 levels fails."""
import numpy as np
import pytest

import oracle
import workloads

H, I, E = 256, 128, 5


def _deq(qw, s, z, N, K, G=128):
    """Independent numpy dequantization of a canonical matrix."""
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2], q[:, 1::2] = qw & 15, qw >> 4
    sc = np.repeat(s.view(np.float16).astype(np.float64), G, axis=1)
    return sc * (q - np.repeat(z.astype(np.int64), G, axis=1))


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _gu(d, x):
    """g, u, S_g, S_u of one expert on activations x [T][H] (numpy fp64)."""
    W = _deq(d["gu_q"], d["gu_s"], d["gu_z"], 2 * I, H)
    gu, S = x @ W.T, np.abs(x) @ np.abs(W).T
    return gu[:, :I], gu[:, I:], S[:, :I], S[:, I:]


def _worst_h(g, u, Sg, Su, c, direction):
    """h' = SiLU(g + a c S_g) (u + b c S_u) with the signs (a, b) that push
    direction * (h' - h) highest, elementwise."""
    best = None
    for a in (-1.0, 1.0):
        for b in (-1.0, 1.0):
            hp = _silu(g + a * c * Sg) * (u + b * c * Su)
            if best is None:
                best = hp
            else:
                better = direction * hp > direction * best
                best = np.where(better, hp, best)
    return best


@pytest.fixture(scope="module")
def layer():
    ex = workloads.moe_experts(21, 0, E, H, I, 0.005, 0.02)
    sh = workloads.moe_shared(21, 0, H, I, 0.005, 0.02)
    x = oracle.widen(workloads.activations(21, 1, 3, H, "bf16"), "bf16")
    return ex, sh, x


def _expert(d, e=None):
    return {k: (v[e] if e is not None else v) for k, v in d.items()}


def _gate_up_canonical(d):
    return d["gu_q"], d["gu_s"], d["gu_z"]


@pytest.mark.parametrize("c,lo,hi", [(1e-7, 1 - 1e-4, 1 + 1e-4), (2e-3, 0.5, 1.0 + 1e-12)])
def test_silu_mul_tolerance_is_the_worst_first_order_change(layer, c, lo, hi):
    ex, _, x = layer
    d = _expert(ex, 1)
    h, tol = oracle.gate_up_silu(x, *_gate_up_canonical(d), I, H, c=c)
    g, u, Sg, Su = _gu(d, x)
    assert np.allclose(h, _silu(g) * u, rtol=1e-12, atol=1e-12 * np.abs(h).max())
    up = np.abs(_worst_h(g, u, Sg, Su, c, 1.0) - h)
    dn = np.abs(_worst_h(g, u, Sg, Su, c, -1.0) - h)
    ratio = np.maximum(up, dn) / tol
    assert ratio.min() >= lo and ratio.max() <= hi, (ratio.min(), ratio.max())


def _moe_worst_change(ex, sh, x, ids, p, c, eps_p, t, n):
    """out'[t][n] - out[t][n] for the perturbation that pushes it up the most."""
    def expert_y(d):
        g, u, Sg, Su = _gu(d, x[t:t + 1])
        Wd = _deq(d["dn_q"], d["dn_s"], d["dn_z"], H, I)[n]
        h = (_silu(g) * u)[0]
        hp = _worst_h(g, u, Sg, Su, c, np.sign(Wd))[0]
        y = Wd @ h
        yp = Wd @ hp + c * np.abs(Wd * h).sum()   # the down linear's own +c sum|w h|
        return y, yp
    out = outp = 0.0
    for j in range(ids.shape[1]):
        y, yp = expert_y(_expert(ex, int(ids[t, j])))
        out += p[t, j] * y
        outp += (p[t, j] + eps_p * np.sign(y)) * yp
    if sh is not None:
        y, yp = expert_y(sh)
        out += y
        outp += yp
    return out, outp - out


@pytest.mark.parametrize("with_shared", [True, False])
def test_moe_tolerance_is_the_worst_first_order_change(layer, with_shared):
    ex, sh, x = layer
    sh = sh if with_shared else None
    ids = np.array([[0, 3], [4, 1], [2, 2 - 1]], dtype=np.int32)
    p = np.array([[0.7, 0.3], [0.55, 0.45], [0.2, 0.8]])
    c, eps_p = 1e-7, 1e-9
    out, tol = oracle.moe(x, ids, p, ex, sh, H, I, E, c=c, eps_p=eps_p)
    for t in range(3):
        for n in (0, 7, 100, H - 1):
            ref, change = _moe_worst_change(ex, sh, x, ids, p, c, eps_p, t, n)
            assert ref == pytest.approx(out[t, n], rel=1e-11, abs=1e-12)
            assert change / tol[t, n] == pytest.approx(1.0, abs=1e-4), (t, n)


def test_moe_tolerance_at_the_workload_factor_is_near_attained(layer):
    ex, sh, x = layer
    ids = np.array([[0, 3], [4, 1], [2, 1]], dtype=np.int32)
    p = np.array([[0.7, 0.3], [0.55, 0.45], [0.2, 0.8]])
    out, tol = oracle.moe(x, ids, p, ex, sh, H, I, E)
    for t in range(3):
        for n in (3, 50, 200):
            _, change = _moe_worst_change(ex, sh, x, ids, p, oracle.C_TOL, oracle.EPS_P, t, n)
            assert 0.5 <= change / tol[t, n] <= 1.0 + 1e-12, (t, n, change / tol[t, n])


# ---- W4A8: the int8 decisions of h that could go either way --------------------------

def _w4a8_expert_h(seed, Hs, Is):
    ex = workloads.moe_experts(seed, 0, 1, Hs, Is, 0.005, 0.02)
    x = workloads.bf16_bits_to_f32(workloads.activations(seed, 1, 1, Hs, "bf16"))
    s_x = float(np.abs(x).max()) / 127.0
    d = _expert(ex, 0)
    xh = oracle.dequant_act(oracle.quantize_act(x, s_x), s_x)   # pinned int8 activations
    W = _deq(d["gu_q"], d["gu_s"], d["gu_z"], 2 * Is, Hs)
    gu = xh @ W.T
    h = (_silu(gu[:, :Is]) * gu[:, Is:])[0]
    Wd = _deq(d["dn_q"], d["dn_s"], d["dn_z"], Hs, Is)
    return ex, x, s_x, h, Wd


def _half_dist(v):
    """Distance of v to the nearest rounding boundary k + 1/2."""
    return np.abs(v - np.floor(v) - 0.5)


@pytest.mark.parametrize("seed", [23, 24, 25])
def test_w4a8_uncertain_decision_term_closed_form(seed):
    """With c = 0, eps_p = 0, top-1 routing to one expert with weight 1 and no
    shared expert, the W4A8 tolerance is only the term for int8 decisions of h
    that could go either way.  Choose the h scale so that h[k0] * r lands on a
    rounding boundary (3.5 steps) while every other h[k] * r stays at least
    1e-3 away from one: exactly decision k0 is uncertain, flipping it moves y[n]
    by one step s_h times |W_d[n][k0]|, so the term is s_h |W_d[:, k0]|.  A
    scale that puts h[k0] at 3.4 steps instead leaves no uncertain decision and
    a zero tolerance."""
    Hs, Is = 256, 128
    ex, x, s_x, h, Wd = _w4a8_expert_h(seed, Hs, Is)
    ids, p = np.zeros((1, 1), np.int32), np.ones((1, 1))
    order = np.argsort(-np.abs(h))
    for k0 in order[:20]:
        for steps, uncertain in ((3.5, True), (3.4, False)):
            s_h = float(np.float32(abs(h[k0]) / steps))
            r = float(np.float32(1.0) / np.float32(s_h))
            others = np.delete(np.abs(h) * r, k0)
            if _half_dist(others).min() < 1e-3 or np.max(others) > 126:
                break
            _, tol = oracle.moe_w4a8(x, s_x, s_h, ids, p, ex, None, Hs, Is, 1, c=0.0,
                                     c_amb=1e-9, eps_p=0.0)
            want = s_h * np.abs(Wd[:, k0]) if uncertain else np.zeros(Hs)
            assert np.allclose(tol[0], want, rtol=1e-12, atol=0.0), (k0, steps)
        else:
            return
    pytest.fail("no activation index with well separated decisions")


def test_w4a8_down_linear_term_is_c_times_its_magnitude():
    """With no uncertain decision (c_amb = 0 and an h scale whose grid keeps
    every h * r away from rounding boundaries), the tolerance of the top-1
    single-expert layer is c times the down projection's magnitude
    sum_k |W_d[n][k] * hhat_k|, hhat = the int8 decision of h times its step."""
    Hs, Is = 256, 128
    ex, x, s_x, h, Wd = _w4a8_expert_h(26, Hs, Is)
    ids, p = np.zeros((1, 1), np.int32), np.ones((1, 1))
    for div in np.linspace(120.0, 127.0, 57):
        s_h = float(np.float32(np.abs(h).max() / div))
        r = np.float32(1.0) / np.float32(s_h)
        v = (h.astype(np.float32) * r).astype(np.float32)
        if _half_dist(v.astype(np.float64)).min() > 1e-3:
            break
    else:
        pytest.fail("no h scale with well separated decisions")
    code = np.clip(np.rint(v), -127, 127).astype(np.float64)
    c = 2e-3
    _, tol = oracle.moe_w4a8(x, s_x, s_h, ids, p, ex, None, Hs, Is, 1, c=c, c_amb=0.0,
                             eps_p=0.0)
    assert np.allclose(tol[0], c * (np.abs(Wd) @ np.abs(code * s_h)), rtol=1e-12, atol=0.0)


# ---- the reference quantizer -----------------------------------------------------------

def test_quantizer_hand_group():
    """One 128-weight group worked by hand (reading R19: min/max with 0 in range,
    15 levels, binary16 scale, rint half to even).
    lo = -0.3, hi = 1.2: scale = fp16(1.5 / 15) = fp16(0.1): 0.1 = 1.6 * 2^-4, the
    significand 0.6 * 1024 = 614.4 rounds to 614, so the bits are (11 << 10) + 614 =
    0x2E66 and the scale is 1638 / 16384 = 0.0999755859375; zero = rint(0.3 / s) =
    rint(3.0007) = 3; codes rint(w / s) + 3: 1.2 -> 12 + 3 = 15, -0.3 -> 0, 0 -> 3,
    0.5 -> 5 + 3 = 8, 0.05 -> rint(0.50012) + 3 = 4, 0.25 -> rint(2.5006) + 3 = 6,
    0.15 -> rint(1.5004) + 3 = 5, -0.149 -> rint(-1.4904) + 3 = 2, 0.1 -> 4.
    With 14 levels the scale would be fp16(0.10714) = 0x2EDB, with 16 levels
    0.09375 = 0x2E00."""
    w = np.full((1, 128), 0.1)
    w[0, :8] = [1.2, -0.3, 0.0, 0.5, 0.05, 0.25, 0.15, -0.149]
    qw, s, z = oracle.quantize(w, 128)
    assert int(s[0, 0]) == 0x2E66
    assert int(z[0, 0]) == 3
    q = oracle.unpack(qw, 1, 128)[0]
    assert q[:8].tolist() == [15, 0, 3, 8, 4, 6, 5, 2]
    assert np.all(q[8:] == 4)


def test_quantizer_hand_group_all_negative():
    """All weights in [-0.75, -0.05]: hi = max(max w, 0) = 0, so the range is
    0.75 and the scale fp16(0.05) = 1.6 * 2^-5 -> (10 << 10) + 614 = 0x2A66
    (0.04998779296875); zero = rint(0.75 / s) = rint(15.0037) = 15; -0.75 -> 0,
    -0.05 -> rint(-1.0002) + 15 = 14, -0.4 -> rint(-8.002) + 15 = 7."""
    w = np.full((1, 128), -0.4)
    w[0, 0], w[0, 1] = -0.75, -0.05
    qw, s, z = oracle.quantize(w, 128)
    assert int(s[0, 0]) == 0x2A66 and int(z[0, 0]) == 15
    q = oracle.unpack(qw, 1, 128)[0]
    assert q[0] == 0 and q[1] == 14 and np.all(q[2:] == 7)
