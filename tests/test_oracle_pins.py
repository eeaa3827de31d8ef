"""Pins for the CPU oracle: each check compares it with something other than itself.

Closed forms, a hand-worked example, brute force, exact invariants and
independent library routines (scipy's erf/ndtr, numpy BLAS products) fix
every function of the oracle, so that a dropped term, a wrong sign, a wrong
index or a transposed operand fails at least one test here.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PHI1 = 0.8413447460685429  # standard normal CDF at 1 (68-95 rule: (1 + 0.6826894921370859)/2)
PHI2 = 0.9772498680518208  # at 2: (1 + 0.9544997361036416)/2


# ---------------------------------------------------------------- GELU
def test_gelu_closed_forms():
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(1.0) == pytest.approx(PHI1, abs=1e-15)
    assert oracle.gelu(-1.0) == pytest.approx(-(1.0 - PHI1), abs=1e-15)
    assert oracle.gelu(2.0) == pytest.approx(2.0 * PHI2, abs=1e-15)
    assert oracle.gelu(12.0) == pytest.approx(12.0, rel=1e-15)       # -> z as z -> +inf
    assert abs(oracle.gelu(-12.0)) < 1e-30                             # -> 0 as z -> -inf
    # odd part: GELU(z) - GELU(-z) = z
    for z in (0.3, 1.7, 4.2):
        assert oracle.gelu(z) - oracle.gelu(-z) == pytest.approx(z, rel=1e-14)


def test_gelu_matches_scipy_ndtr():
    # scipy's normal CDF is an independent implementation (Cephes) of Phi.
    zs = np.linspace(-8, 8, 1601)
    ours = np.array([oracle.gelu(z) for z in zs])
    ref = zs * scipy.special.ndtr(zs)
    assert np.max(np.abs(ours - ref)) < 1e-15 * 8 + 1e-16


def test_gelu_not_tanh_approximation():
    # exact-erf and tanh-approximated GELU differ by ~1e-4 near |z| ~ 2; the oracle is the exact one.
    z = 2.0
    tanh_form = 0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    assert abs(oracle.gelu(z) - tanh_form) > 1e-5
    assert oracle.gelu(z) == pytest.approx(z * scipy.special.ndtr(z), abs=1e-15)


# ---------------------------------------------------------------- routing
def _identity_router(E, d):
    w = np.zeros((E, d), np.float64)
    for e in range(E):
        w[e, e] = 1.0
    return w


def test_zero_router_ties_and_no_renormalisation():
    T, d, E, k = 5, 16, 8, 2
    x = synthetic.normal((T, d), 3, 0, 1.0, "f32").astype(np.float64)
    probs, idx, gate = oracle.route(x, np.zeros((E, d)), k)
    assert np.all(probs == 0.125)
    assert np.all(idx == np.array([0, 1]))          # exact ties go to the lower index
    assert np.all(gate == 0.125)                      # renormalising would give 0.5


def test_softmax_closed_form_ratios():
    # logits = ln(c_e) through an identity router: p_e = c_e / sum(c)
    E = 8
    c = np.array([5.0, 1.0, 7.0, 2.0, 3.0, 8.0, 4.0, 6.0])
    x = np.zeros((1, 16))
    x[0, :E] = np.log(c)
    probs, idx, gate = oracle.route(x, _identity_router(E, 16), 3)
    np.testing.assert_allclose(probs[0], c / c.sum(), rtol=1e-14)
    assert list(idx[0]) == [5, 2, 7]
    np.testing.assert_allclose(gate[0], np.array([8.0, 7.0, 6.0]) / 36.0, rtol=1e-14)


def test_softmax_shift_invariance():
    # a constant feature whose router column is equal for all experts shifts every logit by
    # the same amount and must leave p unchanged
    T, d, E = 16, 32, 8
    x = synthetic.normal((T, d), 5, 0, 1.0, "f32").astype(np.float64)
    w = synthetic.normal((E, d), 5, 1, 0.2, "f32").astype(np.float64)
    w[:, -1] = 0.0
    x[:, -1] = 1.0
    p0, i0, g0 = oracle.route(x, w, 2)
    w2 = w.copy()
    w2[:, -1] = 37.5
    p1, i1, g1 = oracle.route(x, w2, 2)
    np.testing.assert_allclose(p0, p1, rtol=1e-12)
    assert np.array_equal(i0, i1)


def test_identity_router_topk_brute_force():
    rng = np.random.default_rng(11)
    T, d, E = 200, 12, 8
    x = rng.standard_normal((T, d))
    x[5, :E] = [1, 2, 2, 0, -1, 2, 0.5, 0]   # a three-way exact tie at the top
    for k in (1, 2, 3, 8):
        probs, idx, gate = oracle.route(x, _identity_router(E, d), k)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-x[t, e], e))[:k]   # logits are x[:, :E]
            assert list(idx[t]) == order
            z = np.exp(x[t, :E] - x[t, :E].max())
            np.testing.assert_allclose(gate[t], (z / z.sum())[order], rtol=1e-13)
    assert list(oracle.route(x, _identity_router(E, d), 2)[1][5]) == [1, 2]


def test_router_uses_rows_not_columns():
    # a rectangular router with a distinct row per expert: logits = Wr @ x (a numpy product)
    rng = np.random.default_rng(2)
    T, d, E = 30, 10, 4
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((E, d))
    probs, idx, _ = oracle.route(x, w, 1)
    logits = x @ w.T
    ref = np.exp(logits - logits.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(probs, ref, rtol=1e-12)
    assert np.array_equal(idx[:, 0], np.argmax(logits, 1))


def test_route_invariants_decode_shape():
    w = synthetic.make("prefill", T=512, with_weights=False)
    probs, idx, gate = oracle.route(w.x, w.router_w, 2)
    E = w.E
    np.testing.assert_allclose(probs.sum(1), 1.0, atol=1e-12)
    assert np.all(idx[:, 0] != idx[:, 1])
    assert np.all(gate[:, 0] >= gate[:, 1])
    s = gate.sum(1)
    assert np.all(s >= 2.0 / E - 1e-15) and np.all(s <= 1.0)
    assert np.all(s < 1.0)
    np.testing.assert_array_equal(gate, np.take_along_axis(probs, idx.astype(np.int64), 1))
    # the chosen experts carry the two largest probabilities
    srt = -np.sort(-probs, 1)
    np.testing.assert_array_equal(gate, srt[:, :2])


def test_all_28_pairs_at_full_prefill_routing():
    # top-2 of 8 has C(8,2) = 28 expert pairs (book ch. 10, fine-grained expert box);
    # all of them occur over one 8192-token context of the synthetic prefill workload.
    w = synthetic.make("prefill", with_weights=False)
    _, idx, _ = oracle.route(w.x, w.router_w, 2)
    pairs = {tuple(sorted(p)) for p in idx.tolist()}
    assert len(pairs) == 28
    counts = np.bincount(idx.ravel(), minlength=8)
    assert counts.sum() == 2 * 8192 and counts.min() > 1000


def test_skew_workload_shares():
    w = synthetic.make("skew", with_weights=False)
    _, idx, _ = oracle.route(w.x, w.router_w, 2)
    share = np.bincount(idx.ravel(), minlength=8) / idx.size
    assert 0.40 < share[0] < 0.56 and 0.22 < share[1] < 0.38
    assert np.all(share[2:] < 0.08)


def test_renormalisation_negative_control():
    # Mixtral-style renormalisation (book ch. 10, section 10.3.1) must give different outputs
    w = synthetic.make("tiny_f32", T=8, d=32, f=64)
    out, idx, gate = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    renorm = gate / gate.sum(1, keepdims=True)
    out_r = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, renorm)
    assert np.all(gate.sum(1) < 0.999)
    assert np.min(np.abs(out_r - out).max(1) / np.abs(out).max(1)) > 1e-3
    np.testing.assert_allclose(out_r, out / gate.sum(1, keepdims=True), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- permutation
def _brute_permute(idx, E):
    T, k = idx.shape
    pairs = sorted(((int(idx[t, s]), t, s) for t in range(T) for s in range(k)))
    counts = np.bincount(idx.ravel(), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.array([t for (_, t, _) in pairs], np.int32)
    pos = np.zeros((T, k), np.int32)
    for row, (_, t, s) in enumerate(pairs):
        pos[t, s] = row
    return counts, offsets, perm, pos


def _random_routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (7, 8, 2), (300, 8, 2), (64, 4, 1), (50, 8, 8), (33, 64, 8),
                                   (0, 8, 2)])
def test_permute_brute_force(T, E, k):
    rng = np.random.default_rng(T * 131 + E)
    idx = _random_routing(rng, T, E, k)
    c, o, p, pos = oracle.permute(idx, E)
    bc, bo, bp, bpos = _brute_permute(idx, E)
    np.testing.assert_array_equal(c, bc)
    np.testing.assert_array_equal(o, bo)
    np.testing.assert_array_equal(p, bp)
    np.testing.assert_array_equal(pos, bpos)
    # invariants
    assert o[-1] == T * k
    for t in range(T):
        for s in range(k):
            assert p[pos[t, s]] == t
            e = idx[t, s]
            assert o[e] <= pos[t, s] < o[e + 1]
    for e in range(E):
        seg = p[o[e]:o[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_permute_all_on_two_experts_and_empty_experts():
    T, E = 100, 8
    idx = np.tile(np.array([[3, 6]], np.int32), (T, 1))
    idx[::2] = [6, 3]
    c, o, p, pos = oracle.permute(idx, E)
    assert list(c) == [0, 0, 0, T, 0, 0, T, 0]
    np.testing.assert_array_equal(p[o[3]:o[4]], np.arange(T))
    np.testing.assert_array_equal(p[o[6]:o[7]], np.arange(T))


# ---------------------------------------------------------------- expert FFN
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example_E3k2.json")))
    rw = np.array([[math.log(3), 0.0], [math.log(2), 0.0], [0.0, 0.0]])
    x = np.array(g["x"])
    out, idx, gate = oracle.forward(x, rw, np.array(g["w_gate"]), np.array(g["w_up"]), np.array(g["w_down"]), 2)
    assert idx.tolist() == g["expected_idx"]
    np.testing.assert_allclose(gate, g["expected_gate"], rtol=1e-14)
    np.testing.assert_allclose(out, g["expected_out"], rtol=0, atol=g["tolerance"])
    # the derivation's closed form from Phi(1), Phi(2)
    ref = [PHI1 / 2 + 2 * PHI2 / 3, (1 - PHI1) / 2 - 2 * PHI2 / 3]
    np.testing.assert_allclose(out[0], ref, atol=1e-15)


def test_single_expert_reduces_to_dense_geglu_ffn():
    # E=1, k=1: gate = softmax of one logit = 1, so the layer is one dense GeGLU FFN,
    # computed here with numpy BLAS products and scipy's normal CDF.
    rng = np.random.default_rng(4)
    T, d, f = 6, 24, 40
    x = rng.standard_normal((T, d))
    wg, wu, wd = rng.standard_normal((1, f, d)) / 5, rng.standard_normal((1, f, d)) / 5, \
        rng.standard_normal((1, d, f)) / 6
    out, idx, gate = oracle.forward(x, rng.standard_normal((1, d)), wg, wu, wd, 1)
    assert np.all(idx == 0) and np.all(gate == 1.0)
    a = x @ wg[0].T
    b = x @ wu[0].T
    ref = ((a * scipy.special.ndtr(a)) * b) @ wd[0].T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_selector_weights_closed_form():
    # Rectangular 0/1 selector weights (d != f): gate channel j reads input pi_e(j), up channel j
    # reads sigma_e(j), output i reads channel tau_e(i). Then y_i = beta_e * GELU(alpha_e *
    # x[pi(tau(i))]) * x[sigma(tau(i))]. A transposed or mis-indexed operand breaks it.
    rng = np.random.default_rng(9)
    T, d, f, E = 5, 6, 10, 3
    x = rng.standard_normal((T, d))
    pi = [rng.integers(0, d, f) for _ in range(E)]
    sg = [rng.integers(0, d, f) for _ in range(E)]
    tau = [rng.integers(0, f, d) for _ in range(E)]
    alpha = [0.5, 2.0, -1.0]
    beta = [1.0, -3.0, 0.25]
    wg = np.zeros((E, f, d)); wu = np.zeros((E, f, d)); wd = np.zeros((E, d, f))
    for e in range(E):
        for j in range(f):
            wg[e, j, pi[e][j]] = alpha[e]
            wu[e, j, sg[e][j]] = 1.0
        for i in range(d):
            wd[e, i, tau[e][i]] = beta[e]
    # zero router: experts (0, 1), gates (1/3, 1/3)
    out, idx, gate = oracle.forward(x, np.zeros((E, d)), wg, wu, wd, 2)
    assert np.all(idx == [0, 1]) and np.allclose(gate, 1 / 3, rtol=1e-15)
    for t in range(T):
        for i in range(d):
            ref = 0.0
            for e in (0, 1):
                j = tau[e][i]
                z = alpha[e] * x[t, pi[e][j]]
                ref += (1 / 3) * beta[e] * (z * scipy.special.ndtr(z)) * x[t, sg[e][j]]
            assert out[t, i] == pytest.approx(ref, rel=1e-13, abs=1e-15)


def test_identity_weights_closed_form():
    # d = f, Wg = Wu = Wd = I for every expert: out = (g0 + g1) * GELU(x) * x
    rng = np.random.default_rng(5)
    T, d, E = 9, 16, 8
    x = rng.standard_normal((T, d))
    eye = np.broadcast_to(np.eye(d), (E, d, d)).copy()
    rw = rng.standard_normal((E, d)) / 4
    out, idx, gate = oracle.forward(x, rw, eye, eye, eye, 2)
    ref = gate.sum(1, keepdims=True) * (x * scipy.special.ndtr(x)) * x
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("E,k,wdt", [(1, 1, "f64"), (2, 1, "f32"), (2, 2, "bf16"), (8, 2, "f32"), (8, 2, "bf16"),
                                     (8, 1, "i8"), (8, 2, "i8")])
def test_sparse_equals_dense_onehot(E, k, wdt):
    # the pages' own dense formulation (all experts, one-hot mask) as brute force
    T, d, f = 24, 32, 48
    act = "bf16" if wdt in ("bf16", "i8") else "f32"
    w = synthetic.make("tiny_f32", T=T, d=d, f=f, E=E, k=k, act_dtype=act, w_dtype="f32" if wdt == "f64" else wdt)
    sc = synthetic.random_scales(E, d, f, 1) if wdt == "i8" else None
    args = [w.w_gate, w.w_up, w.w_down]
    if wdt == "f64":
        args = [a.astype(np.float64) for a in args]
    out, _, _ = oracle.forward(w.x, w.router_w, *args, k, scales=sc)
    dense = oracle.dense_onehot(w.x, w.router_w, *args, k, scales=sc)
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-14 * np.abs(out).max())


def test_exact_power_of_two_scaling():
    w = synthetic.make("tiny_f32", T=16, d=32, f=64)
    out, _, _ = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    out_d, _, _ = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, 2 * w.w_down, 2)
    out_u, _, _ = oracle.forward(w.x, w.router_w, w.w_gate, 4 * w.w_up, w.w_down, 2)
    np.testing.assert_array_equal(out_d, 2 * out)
    np.testing.assert_array_equal(out_u, 4 * out)
    # scaling the gate branch is NOT linear (GELU)
    out_g, _, _ = oracle.forward(w.x, w.router_w, 2 * w.w_gate, w.w_up, w.w_down, 2)
    assert np.abs(out_g - 2 * out).max() > 1e-3 * np.abs(out).max()


def test_token_permutation_equivariance():
    w = synthetic.make("tiny_f32", T=20, d=32, f=64)
    out, idx, gate = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    perm = np.random.default_rng(1).permutation(20)
    out_p, idx_p, gate_p = oracle.forward(w.x[perm], w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    np.testing.assert_array_equal(out_p, out[perm])
    np.testing.assert_array_equal(idx_p, idx[perm])


def test_expert_relabelling_invariance():
    w = synthetic.make("tiny_f32", T=20, d=32, f=64)
    out, idx, gate = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    rl = np.array([3, 7, 0, 5, 1, 6, 2, 4])   # new expert e is old expert rl[e]
    out_r, idx_r, gate_r = oracle.forward(w.x, w.router_w[rl], w.w_gate[rl], w.w_up[rl], w.w_down[rl], 2)
    np.testing.assert_array_equal(rl[idx_r], idx)
    # the softmax denominator sums the experts in a different order, so equal up to rounding
    np.testing.assert_allclose(out_r, out, rtol=1e-13, atol=1e-15)


def test_int8_scales_are_per_output_channel():
    # q * s with distinct per-channel scales equals the same layer on pre-multiplied f64 weights
    # (q * s is exact in double), which pins which channel each scale belongs to.
    T, d, f, E = 12, 32, 48, 4
    w = synthetic.make("int8", T=T, d=d, f=f, E=E)
    s = synthetic.random_scales(E, d, f, 3).astype(np.float64)
    sg = s[:E * f].reshape(E, f, 1)
    su = s[E * f:2 * E * f].reshape(E, f, 1)
    sd = s[2 * E * f:].reshape(E, d, 1)
    out8, _, _ = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2, scales=s.astype(np.float32))
    out64, _, _ = oracle.forward(w.x, w.router_w, w.w_gate * sg, w.w_up * su, w.w_down * sd, 2)
    np.testing.assert_allclose(out8, out64, rtol=1e-14, atol=1e-300)
    # the transposed reading of the down scales gives a different layer
    bad = np.concatenate([s[:2 * E * f], s[2 * E * f:][::-1]]).astype(np.float32)
    out_bad, _, _ = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2, scales=bad)
    assert np.abs(out_bad - out8).max() > 1e-3 * np.abs(out8).max()


def test_int8_integer_exact_projection():
    # scales = 1 and small integer activations: a and b are exact integers, h is computed from them
    T, d, f, E = 3, 8, 8, 2
    rng = np.random.default_rng(8)
    x = rng.integers(-3, 4, (T, d)).astype(np.float64)
    qg = rng.integers(-127, 128, (E, f, d)).astype(np.int8)
    qu = rng.integers(-127, 128, (E, f, d)).astype(np.int8)
    qd = rng.integers(-127, 128, (E, d, f)).astype(np.int8)
    ones = np.ones(2 * E * f + E * d, np.float32)
    for t in range(T):
        for e in range(E):
            y = oracle.expert(x, t, e, qg, qu, qd, scales=ones)
            a = qg[e].astype(np.int64) @ x[t].astype(np.int64)
            b = qu[e].astype(np.int64) @ x[t].astype(np.int64)
            h = (a * scipy.special.ndtr(a)) * b
            ref = qd[e].astype(np.float64) @ h
            np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-9)


def test_bf16_inputs_widen_exactly():
    w = synthetic.make("tiny_f32", T=8, d=32, f=64, act_dtype="bf16", w_dtype="bf16")
    wide = [synthetic.bf16_bits_to_f32(a) for a in (w.x, w.router_w, w.w_gate, w.w_up, w.w_down)]
    o1, i1, g1 = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    o2, i2, g2 = oracle.forward(*wide, 2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(i1, i2)


def test_token_subset_matches_full():
    w = synthetic.make("tiny_f32", T=16, d=32, f=64)
    out, idx, gate = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2)
    sub = [15, 0, 7]
    o = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, gate, tokens=sub)
    np.testing.assert_array_equal(o, out[sub])


def test_oracle_rejects_bad_arguments():
    with pytest.raises(RuntimeError):
        oracle.route(np.zeros((2, 4)), np.zeros((3, 4)), 4)          # k > E
    with pytest.raises(RuntimeError):
        oracle.permute(np.array([[0, 9]], np.int32), 8)               # expert index out of range
