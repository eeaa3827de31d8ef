"""Pins for the oracle's layer variants: SiLU experts, renormalised gates,
capacity-factor drops, the sandwich sub-layer (RMSNorm before and after the
MoE, plus the residual), and the fine-grained layout (hundreds of experts, a
per-expert selection bias, shared experts).

As in test_oracle_pins.py, every check compares the oracle with something
other than itself: closed forms, brute force written here with numpy/scipy
primitives, exact invariants, or an independent library (torch's bf16
rounding, scipy's expit and ndtr).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synthetic


def _f64(a):
    a = np.asarray(a)
    return synthetic.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _bf16_bits(v):
    return synthetic.f32_to_bf16_bits(np.asarray(v, np.float32))


# ---------------------------------------------------------------- SiLU
def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), abs=1e-16)
    assert oracle.silu(1.0) == pytest.approx(0.7310585786300049, abs=1e-16)  # logistic(1)
    # odd part: sigmoid(z) + sigmoid(-z) = 1, so SiLU(z) - SiLU(-z) = z
    for z in (0.3, 1.7, 4.2, 11.0):
        assert oracle.silu(z) - oracle.silu(-z) == pytest.approx(z, rel=1e-14)
    # tanh form: z sigmoid(z) = z (1 + tanh(z/2)) / 2
    for z in np.linspace(-6, 6, 25):
        assert oracle.silu(z) == pytest.approx(0.5 * z * (1.0 + math.tanh(0.5 * z)), abs=1e-15)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)


def test_silu_matches_scipy_expit():
    zs = np.linspace(-20, 20, 801)
    ours = np.array([oracle.silu(z) for z in zs])
    np.testing.assert_allclose(ours, zs * scipy.special.expit(zs), rtol=1e-14, atol=1e-300)


def test_silu_and_gelu_tails_differ_as_the_pages_say():
    # SiLU keeps a small negative output far left, GELU is practically zero there
    assert oracle.silu(-10.0) == pytest.approx(-10.0 / (1.0 + math.exp(10.0)), rel=1e-13)
    assert -5e-4 < oracle.silu(-10.0) < -4e-4
    assert abs(oracle.gelu(-10.0)) < 1e-20


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rne_ties_to_even_and_exact_values():
    assert oracle.bf16_rne(1.0) == 0x3F80
    assert oracle.bf16_rne(-2.0) == 0xC000
    assert oracle.bf16_rne(0.0) == 0x0000
    assert oracle.bf16_rne(-0.0) == 0x8000
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to the even one (1)
    assert oracle.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is the midpoint of 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6 (even mantissa)
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above a midpoint rounds up, just below rounds down
    assert oracle.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8 - 2.0 ** -40) == 0x3F81
    # carry into the exponent
    assert oracle.bf16_rne(2.0 - 2.0 ** -9) == 0x4000


def test_bf16_rne_matches_torch_on_float32_values():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ours = np.array([oracle.bf16_rne(float(a)) for a in v], dtype=np.uint16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


# ---------------------------------------------------------------- renormalised gates
def test_renormalised_zero_router_and_k1():
    x = synthetic.normal((5, 64), 0, 0, 1.0, "bf16")
    wr = np.zeros((8, 64), np.uint16)
    _, idx, gate = oracle.route_v(x, wr, 2, renormalize=True)
    assert (idx == [0, 1]).all()
    assert (gate == 0.5).all()
    wr = synthetic.normal((8, 64), 0, 1, 0.125, "bf16")
    _, idx, gate = oracle.route_v(x, wr, 1, renormalize=True)
    assert (gate == 1.0).all()


def test_renormalised_gates_are_softmax_of_selected_logits():
    w = synthetic.make("decode", T=96, d=512, with_weights=False)
    _, idx0, gate0 = oracle.route_v(w.x, w.router_w, 2, renormalize=False)
    _, idx, gate = oracle.route_v(w.x, w.router_w, 2, renormalize=True)
    # renormalising does not change which experts are chosen
    np.testing.assert_array_equal(idx, idx0)
    np.testing.assert_allclose(gate.sum(axis=1), 1.0, atol=1e-15)
    logits = _f64(w.x) @ _f64(w.router_w).T          # numpy BLAS, independent of the oracle's loop
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(gate, scipy.special.softmax(sel, axis=1), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- capacity
def test_capacity_values():
    assert oracle.capacity(1.0, 2048, 8, 2) == 512
    assert oracle.capacity(1.25, 8, 8, 2) == 2          # floor(2.5)
    assert oracle.capacity(2.0, 8, 8, 2) == 4
    assert oracle.capacity(0.01, 8, 8, 2) == 0
    assert oracle.capacity(0.0, 8, 8, 2) == -1          # no cap
    assert oracle.capacity(-1.0, 8, 8, 2) == -1


def _brute_permute_cap(idx, E, cap):
    T, k = idx.shape
    kept = {e: [t for t in range(T) if e in idx[t]] for e in range(E)}
    if cap >= 0:
        kept = {e: ts[:cap] for e, ts in kept.items()}
    counts = np.array([len(kept[e]) for e in range(E)], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.zeros(T * k, np.int32)
    pos = np.full((T, k), -1, np.int32)
    for e in range(E):
        for r, t in enumerate(kept[e]):
            perm[offsets[e] + r] = t
            pos[t, list(idx[t]).index(e)] = offsets[e] + r
    return counts, offsets, perm, pos


@pytest.mark.parametrize("T,E,k,cap", [(1, 4, 2, 0), (17, 8, 2, 3), (40, 8, 2, 10), (33, 5, 3, 7), (50, 8, 1, 4),
                                       (12, 8, 2, -1), (12, 8, 2, 100)])
def test_permute_cap_brute_force(T, E, k, cap):
    rng = np.random.default_rng(T * 131 + E * 7 + k + cap)
    # skewed draws so that some experts overflow
    pw = np.array([8.0, 4.0] + [1.0] * (E - 2))[:E]
    idx = np.stack([rng.choice(E, size=k, replace=False, p=pw / pw.sum()) for _ in range(T)]).astype(np.int32)
    got = oracle.permute_cap(idx, E, cap)
    exp = _brute_permute_cap(idx, E, cap)
    for g, e in zip(got[:2], exp[:2]):
        np.testing.assert_array_equal(g, e)
    n = int(exp[1][-1])
    np.testing.assert_array_equal(got[2][:n], exp[2][:n])
    np.testing.assert_array_equal(got[3], exp[3])
    if cap >= 0:
        assert (got[0] <= cap).all()


def test_permute_cap_without_cap_equals_permute():
    w = synthetic.make("decode", T=200, d=256, with_weights=False)
    _, idx, _ = oracle.route(w.x, w.router_w, 2)
    a = oracle.permute(idx, 8)
    b = oracle.permute_cap(idx, 8, -1)
    c = oracle.permute_cap(idx, 8, 400)
    for x, y, z in zip(a, b, c):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(x, z)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    one = np.ones(4)
    # constant rows c*1, eps = 0: every output is sign(c) times the weight
    v = np.array([[2.5] * 4, [-0.75] * 4])
    np.testing.assert_allclose(oracle.rmsnorm(v, one, 0.0), [[1.0] * 4, [-1.0] * 4], atol=1e-15)
    # (3, 4): mean square 12.5
    out = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    np.testing.assert_allclose(out, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    # eps adds under the root: (3, 4) with eps 0.5 -> divide by sqrt(13)
    out = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.5)
    np.testing.assert_allclose(out, [[3 / math.sqrt(13.0), 4 / math.sqrt(13.0)]], rtol=1e-15)
    # the weight scales each channel on its own
    out = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.array([2.0, -0.5]), 0.0)
    np.testing.assert_allclose(out, [[6 / math.sqrt(12.5), -2 / math.sqrt(12.5)]], rtol=1e-15)
    # zero row stays zero (0 / sqrt(eps))
    assert (oracle.rmsnorm(np.zeros((1, 8)), np.ones(8), 1e-5) == 0.0).all()


def test_rmsnorm_invariants():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((6, 300))
    g = np.ones(300)
    a = oracle.rmsnorm(v, g, 0.0)
    np.testing.assert_allclose((a ** 2).mean(axis=1), 1.0, rtol=1e-14)         # unit mean square
    np.testing.assert_allclose(oracle.rmsnorm(37.5 * v, g, 0.0), a, rtol=1e-13)  # scale invariance
    np.testing.assert_allclose(oracle.rmsnorm(-v, g, 0.0), -a, rtol=1e-15)      # odd


# ---------------------------------------------------------------- whole layer with variants
def _brute_dense_layer(w, act, renorm, cap, tokens=None):
    """Every expert on every token with numpy products, then one-hot(kept top-k) * gate, plus the
    shared experts (after the routed ones in the weights) with gate 1."""
    x = _f64(w.x)
    wr = _f64(w.router_w)
    logits = x @ wr.T
    p = scipy.special.softmax(logits, axis=1)
    key = p if w.router_bias is None else p + w.router_bias.astype(np.float64)[None, :]
    order = np.lexsort((np.arange(w.E)[None, :].repeat(w.T, 0), -key), axis=1)  # key (-(p + b), e)
    idx = order[:, :w.k]
    gate = np.take_along_axis(p, idx, axis=1)
    if renorm:
        gate = gate / gate.sum(axis=1, keepdims=True)
    keep = np.ones_like(idx, bool)
    if cap >= 0:
        used = np.zeros(w.E, int)
        for t in range(w.T):
            for s in range(w.k):
                e = idx[t, s]
                keep[t, s] = used[e] < cap
                used[e] += 1
    fn = (lambda z: z * scipy.special.expit(z)) if act == "silu" else (lambda z: z * scipy.special.ndtr(z))
    out = np.zeros((w.T, w.d))
    for e in range(w.E):
        a = x @ _f64(w.w_gate[e]).T
        b = x @ _f64(w.w_up[e]).T
        y = (fn(a) * b) @ _f64(w.w_down[e]).T
        m = np.where((idx == e) & keep, gate, 0.0).sum(axis=1)
        out += m[:, None] * y
    for j in range(w.n_shared):
        e = w.E + j
        a = x @ _f64(w.w_gate[e]).T
        b = x @ _f64(w.w_up[e]).T
        out += (fn(a) * b) @ _f64(w.w_down[e]).T
    return out, idx, gate, keep


def _layer(w, **kw):
    return oracle.layer(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, w.k, scales=w.scales,
                        activation=oracle.SILU if w.activation == "silu" else oracle.GELU,
                        renormalize=w.renormalize, capacity_factor=w.capacity_factor,
                        norm_pre=w.norm_pre, norm_post=w.norm_post, norm_eps=w.norm_eps, n_shared=w.n_shared,
                        router_bias=w.router_bias, **kw)


def test_layer_with_variants_off_equals_forward():
    w = synthetic.make("tiny_f32", T=24, d=64, f=128)
    r = _layer(w)
    out, idx, gate = oracle.forward(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, w.k)
    np.testing.assert_array_equal(r["out"], out)
    np.testing.assert_array_equal(r["idx"], idx)
    assert r["u"] is None


@pytest.mark.parametrize("act,renorm,cf", [("silu", True, 0.0), ("silu", False, 0.0), ("gelu", True, 0.0),
                                           ("gelu", False, 0.75), ("silu", True, 0.5)])
def test_layer_variants_match_dense_brute_force(act, renorm, cf):
    w = synthetic.make("tiny_f32", T=32, d=64, f=96, activation=act, renormalize=renorm, capacity_factor=cf,
                       skew=cf > 0)
    r = _layer(w)
    cap = oracle.capacity(cf, w.T, w.E, w.k)
    ref, idx, gate, keep = _brute_dense_layer(w, act, renorm, cap)
    np.testing.assert_array_equal(r["idx"][:, :w.k], idx)
    np.testing.assert_allclose(r["gate"][:, :w.k], gate, rtol=1e-12)
    np.testing.assert_array_equal(r["pos"][:, :w.k] >= 0, keep)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)
    if cf > 0:
        assert (~keep).any(), "the skewed workload must overflow at this capacity"


def test_capacity_zero_drops_everything():
    w = synthetic.make("tiny_f32", T=16, d=64, f=96, capacity_factor=0.01)
    r = _layer(w)
    assert (r["pos"] == -1).all()
    assert (r["out"] == 0.0).all()
    ws = synthetic.make("tiny_f32", T=16, d=64, f=96, capacity_factor=0.01, sandwich=True)
    r = _layer(ws)
    np.testing.assert_array_equal(r["out"], _f64(ws.x))          # dropped tokens ride the residual


def test_sandwich_zero_experts_is_the_residual():
    w = synthetic.make("decode", T=12, d=256, f=256, sandwich=True)
    w.w_down = np.zeros_like(w.w_down)
    r = _layer(w)
    np.testing.assert_array_equal(r["out"], _f64(w.x))


def _identity_workload(act, eps):
    d = 128
    w = synthetic.make("decode", T=20, d=d, f=d, activation=act, sandwich=True, norm_eps=eps)
    eye = _bf16_bits(np.eye(d))
    w.w_gate = np.ascontiguousarray(np.broadcast_to(eye, (w.E, d, d)))
    w.w_up = w.w_gate.copy()
    w.w_down = w.w_gate.copy()
    return w


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_sandwich_identity_experts_closed_form(act):
    # identity experts: the MoE output is (g0 + g1) * act(u) * u, and with eps = 0 the
    # post-norm removes the gate sum: out = x + g_post * v / rms(v), v = act(u) * u
    w = _identity_workload(act, 0.0)
    r = _layer(w)
    x = _f64(w.x)
    rms = np.sqrt((x ** 2).mean(axis=1, keepdims=True))
    u_exact = x / rms * _f64(w.norm_pre)[None, :]
    u_bits = np.array([[oracle.bf16_rne(v) for v in row] for row in u_exact], np.uint16)
    np.testing.assert_array_equal(r["u"], u_bits)
    u = _f64(u_bits)
    fn = scipy.special.expit if act == "silu" else scipy.special.ndtr
    v = u * fn(u) * u
    ref = x + _f64(w.norm_post)[None, :] * v / np.sqrt((v ** 2).mean(axis=1, keepdims=True))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_sandwich_single_expert_is_a_dense_normed_ffn():
    w = synthetic.make("decode", T=10, d=256, f=384, E=1, k=1, sandwich=True, norm_eps=1e-5)
    r = _layer(w)
    x = _f64(w.x)
    u = _f64(r["u"])
    # u is the bf16 rounding of the pre-norm (checked bitwise above); the FFN by numpy products
    y = ((u @ _f64(w.w_gate[0]).T) * scipy.special.ndtr(u @ _f64(w.w_gate[0]).T) * (u @ _f64(w.w_up[0]).T)) \
        @ _f64(w.w_down[0]).T
    ref = x + _f64(w.norm_post)[None, :] * y / np.sqrt((y ** 2).mean(axis=1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-11, atol=1e-11)


def test_sandwich_post_norm_absorbs_expert_output_scale():
    # the post-norm is what bounds the un-normalised gates' output scale: doubling the
    # down projection (exact in bf16) leaves the sub-layer output unchanged when eps = 0
    w = synthetic.make("decode", T=16, d=256, f=256, sandwich=True, norm_eps=0.0)
    a = _layer(w)["out"]
    w.w_down = _bf16_bits(2.0 * synthetic.bf16_bits_to_f32(w.w_down))
    b = _layer(w)["out"]
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-13)
    # without the norms the same change doubles the MoE output
    w2 = synthetic.make("decode", T=16, d=256, f=256)
    c = _layer(w2)["out"]
    w2.w_down = _bf16_bits(2.0 * synthetic.bf16_bits_to_f32(w2.w_down))
    np.testing.assert_allclose(_layer(w2)["out"], 2.0 * c, rtol=1e-13)


def test_sandwich_routes_on_the_normed_input():
    # the router sees u, not x: scaling x by 2 (exact) does not change u with eps = 0,
    # so the routing and the MoE output are unchanged and only the residual doubles
    w = synthetic.make("decode", T=16, d=256, f=256, sandwich=True, norm_eps=0.0)
    a = _layer(w)
    x2 = _bf16_bits(2.0 * synthetic.bf16_bits_to_f32(w.x))
    w.x = x2
    b = _layer(w)
    np.testing.assert_array_equal(a["u"], b["u"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(b["out"] - _f64(x2), a["out"] - _f64(x2) / 2.0, rtol=1e-12, atol=1e-12)


def test_sampled_tokens_match_full_layer_with_variants():
    w = synthetic.make("tiny_f32", T=40, d=64, f=96, activation="silu", renormalize=True, capacity_factor=0.6,
                       skew=True, sandwich=True)
    full = _layer(w)["out"]
    toks = [39, 0, 17, 5]
    part = _layer(w, tokens=toks)["out"]
    np.testing.assert_array_equal(part, full[toks])


def test_layer_rejects_bad_arguments():
    w = synthetic.make("tiny_f32", T=4, d=64, f=96)
    with pytest.raises(RuntimeError):
        oracle.layer(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2, activation=7)
    with pytest.raises(RuntimeError):
        oracle.layer(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, 2, norm_pre=np.ones(64, np.float32),
                     norm_post=np.ones(64, np.float32), norm_eps=-1.0)


# ---------------------------------------------------------------- fine-grained: many experts, bias, shared experts
def test_selection_bias_on_equal_probabilities():
    # zero router: every p = 1/E, so the bias alone decides the choice (ties to the lower index),
    # and the gates stay the probabilities: 1/E each, 1/k after renormalisation
    E, k = 32, 4
    x = synthetic.normal((6, 64), 0, 0, 1.0, "bf16")
    wr = np.zeros((E, 64), np.uint16)
    b = np.zeros(E, np.float32)
    b[[5, 17, 30]] = [0.3, 0.2, 0.1]
    b[[9, 2]] = 0.05
    _, idx, gate = oracle.route_v(x, wr, k, renormalize=False, bias=b)
    assert (idx == [5, 17, 30, 2]).all()                 # 2 before 9 at equal bias
    np.testing.assert_allclose(gate, 1.0 / E, rtol=1e-15)
    _, idx, gate = oracle.route_v(x, wr, k, renormalize=True, bias=b)
    np.testing.assert_allclose(gate, 1.0 / k, rtol=1e-15)


def test_selection_bias_forces_an_expert_but_not_its_gate():
    w = synthetic.make("decode", T=40, d=256, E=16, k=2, with_weights=False)
    b = np.zeros(16, np.float32)
    b[11] = 10.0
    probs, idx, gate = oracle.route_v(w.x, w.router_w, 2, bias=b)
    assert (idx[:, 0] == 11).all()
    np.testing.assert_array_equal(gate[:, 0], probs[:, 11])   # the gate is the unbiased probability
    _, idx0, _ = oracle.route_v(w.x, w.router_w, 2)
    np.testing.assert_array_equal(idx[:, 1], np.where(idx0[:, 0] == 11, idx0[:, 1], idx0[:, 0]))


@pytest.mark.parametrize("E,k,bias", [(256, 8, True), (256, 8, False), (160, 6, True), (512, 3, False)])
def test_many_expert_routing_brute_force(E, k, bias):
    w = synthetic.make("dsv3_decode", T=48, d=256, E=E, k=k, with_weights=False, router_bias=bias)
    probs, idx, gate = oracle.route_v(w.x, w.router_w, k, renormalize=True, bias=w.router_bias)
    p = scipy.special.softmax(_f64(w.x) @ _f64(w.router_w).T, axis=1)
    np.testing.assert_allclose(probs, p, rtol=1e-12, atol=1e-18)
    key = p if w.router_bias is None else p + w.router_bias.astype(np.float64)
    order = np.lexsort((np.arange(E)[None, :].repeat(w.T, 0), -key), axis=1)[:, :k]
    np.testing.assert_array_equal(idx, order)
    sel = np.take_along_axis(p, order, axis=1)
    np.testing.assert_allclose(gate, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)


def test_capacity_spares_shared_experts():
    idx = np.array([[0, 4], [0, 4], [0, 4], [1, 4]], np.int32)   # expert 4 is the shared one (E_cap = 4)
    c, o, p, pos = oracle.permute_cap(idx, 5, 1, E_cap=4)
    assert list(c) == [1, 1, 0, 0, 4]
    assert (pos[:, 1] >= 0).all() and list(pos[:, 0]) == [0, -1, -1, 1]


@pytest.mark.parametrize("act,renorm,cf,bias", [("silu", True, 0.0, True), ("gelu", False, 0.0, False),
                                                ("silu", True, 0.6, True)])
def test_shared_expert_layer_matches_dense_brute_force(act, renorm, cf, bias):
    w = synthetic.make("dsv3_decode", T=24, d=64, f=96, E=16, k=4, activation=act, renormalize=renorm,
                       capacity_factor=cf, router_bias=bias, act_dtype="f32", w_dtype="f32")
    assert w.n_shared == 1 and w.w_gate.shape[0] == 17
    r = _layer(w)
    assert r["idx"].shape == (24, 5)
    assert (r["idx"][:, 4] == 16).all() and (r["gate"][:, 4] == 1.0).all() and (r["pos"][:, 4] >= 0).all()
    cap = oracle.capacity(cf, w.T, w.E, w.k)
    ref, idx, gate, keep = _brute_dense_layer(w, act, renorm, cap)
    np.testing.assert_array_equal(r["idx"][:, :4], idx)
    np.testing.assert_allclose(r["gate"][:, :4], gate, rtol=1e-12)
    np.testing.assert_array_equal(r["pos"][:, :4] >= 0, keep)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def test_shared_expert_alone_is_a_dense_ffn():
    # routed experts' down projections zero: the layer is the shared expert's SwiGLU FFN on every token
    w = synthetic.make("dsv3_decode", T=10, d=128, f=64, E=8, k=2)
    w.w_down = w.w_down.copy()
    w.w_down[:8] = 0
    r = _layer(w)
    x = _f64(w.x)
    a = x @ _f64(w.w_gate[8]).T
    y = (a * scipy.special.expit(a) * (x @ _f64(w.w_up[8]).T)) @ _f64(w.w_down[8]).T
    np.testing.assert_allclose(r["out"], y, rtol=1e-12, atol=1e-14)
