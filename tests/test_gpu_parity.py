"""GPU parity of the HIP path against the CPU oracle, at sizes the oracle finishes in
seconds (several tiles plus ragged tails), through the C ABI.

Routing: indices equal the oracle's (a differing token is allowed only where the
two probabilities are within 1e-6, and must then still be a valid top-k); GPU
gates equal the oracle probabilities to fp32 rounding. Permutation: bit-exact
against the oracle's permutation of the GPU routing. Output: per-token normwise
relative error against the oracle evaluated on the GPU's routing, 2e-2 for bf16,
5e-2 for 8-bit weights, 1e-4 for fp32.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import TOL, check_permutation, check_routing, dev_workload, elementwise_err, normwise_err, run_layer

torch = pytest.importorskip("torch")
import mixture_experts_transformer_gemm_amd as gm  # noqa: E402

pytestmark = pytest.mark.gpu


def _full_check(w, scales=None, expect_exact_routing=True):
    if scales is not None:
        w.scales = scales
    got, dbg = run_layer(w, torch)
    probs, oidx, _ = oracle.route(w.x, w.router_w, w.k)
    check_routing(dbg["idx"], dbg["gate"], probs)
    if expect_exact_routing:
        np.testing.assert_array_equal(dbg["idx"], oidx)
    check_permutation(dbg["idx"], dbg, w.E)
    gates = np.take_along_axis(probs, dbg["idx"].astype(np.int64), 1)
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, dbg["idx"], gates, scales=w.scales)
    err = normwise_err(got, ref)
    tol = TOL["f32" if w.act_dtype == "f32" else ("i8" if w.w_dtype == "i8" else "bf16")]
    assert err <= tol, f"normwise error {err:.3e} > {tol}"
    assert np.all(np.isfinite(got))
    return got, dbg, err


@pytest.mark.parametrize("T", [1, 5, 8, 16, 24, 32, 37, 63, 64, 65, 100, 128, 129, 257, 300, 777, 2049])
def test_bf16_layer_small(T):
    w = synthetic.make("decode", T=T, d=256, f=512, seed=T)
    _full_check(w)


@pytest.mark.parametrize("T,d,f", [(3, 512, 256), (48, 512, 768), (200, 512, 768), (300, 768, 1280), (600, 256, 256),
                                   (1500, 512, 768), (2600, 768, 1280)])
def test_bf16_layer_other_shapes(T, d, f):
    w = synthetic.make("decode", T=T, d=d, f=f, seed=100 + T)
    _full_check(w)


@pytest.mark.parametrize("T", [3, 24, 40, 128, 200, 513, 1600, 2049, 4100])
def test_int8_layer_small_random_scales(T):
    # distinct per-channel scales pin which output channel each scale belongs to
    w = synthetic.make("int8", T=T, d=256, f=512, seed=T)
    _full_check(w, scales=synthetic.random_scales(w.E, w.d, w.f, seed=T))


def test_tiny_f32_workload():
    # the tiny fp32 workload exactly as specified: T=64, d=256, E=8, top-2, f=1024, seed 0
    w = synthetic.make("tiny_f32")
    _full_check(w)


@pytest.mark.parametrize("T,d,f", [(1, 8, 4), (7, 24, 20), (33, 64, 96), (301, 64, 96)])
def test_f32_layer_odd_shapes(T, d, f):
    w = synthetic.make("tiny_f32", T=T, d=d, f=f, seed=T)
    _full_check(w)


# (16, 4, 2100) and (64, 8, 4200): about 525 rows per expert, so the ping-pong kernel runs with
# 16 and 64 experts of two 320-row tiles each, a full and a partial one, spread over the per-XCD
# tile ranges; (16, 4, 1200) and (64, 8, 2400): about 300 rows per expert, mostly one partial tile
@pytest.mark.parametrize("E,k,T", [(1, 1, 20), (4, 1, 50), (2, 2, 9), (16, 4, 60), (64, 8, 50), (16, 4, 260),
                                   (1, 1, 700), (2, 1, 333), (64, 8, 300), (32, 2, 5000), (16, 4, 2100),
                                   (64, 8, 4200), (16, 4, 1200), (64, 8, 2400)])
def test_expert_and_k_variants(E, k, T):
    w = synthetic.make("decode", T=T, d=256, f=256, E=E, k=k, seed=E * 10 + k)
    _full_check(w)


@pytest.mark.parametrize("T", [100, 300])
def test_routing_override_imbalanced(T):
    # every token on experts 3 and 6 (all other experts empty), slot order alternating,
    # gates chosen by the caller (a sum above 1 is fine for the kernels)
    w = synthetic.make("decode", T=T, d=256, f=512, seed=7)
    idx = np.tile(np.array([[3, 6]], np.int32), (T, 1))
    idx[1::2] = [6, 3]
    gate = np.tile(np.array([[0.7, 0.45]], np.float32), (T, 1))
    got, dbg = run_layer(w, torch, route_idx=idx, route_gate=gate)
    np.testing.assert_array_equal(dbg["idx"], idx)
    check_permutation(idx, dbg, w.E)
    assert list(dbg["counts"]) == [0, 0, 0, T, 0, 0, T, 0]
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, gate.astype(np.float64))
    assert normwise_err(got, ref) <= TOL["bf16"]


# Expert segments of 5, 6, 9 and 10 row tiles of 320 rows: the ping-pong kernel walks an expert's
# row tiles in groups of 4, then the remainder (4 + 1, 4 + 2, 4 + 4 + 1, 4 + 4 + 2), here next to an
# empty expert, a one-row expert, one exact tile and one tile plus a row, through a caller routing
# with k = 1 and per-token gates.
def test_pingpong_tile_groups_with_remainders():
    counts = [1500, 1800, 0, 2600, 1, 3000, 320, 321]
    T = sum(counts)
    w = synthetic.make("decode", T=T, d=256, f=512, k=1, seed=11)
    dev = dev_workload(w, torch)
    assert gm.grok_moe_tile_rows(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], k=1) == 320
    rng = np.random.default_rng(3)
    idx = np.repeat(np.arange(w.E, dtype=np.int32), counts)[rng.permutation(T)][:, None]
    gate = rng.uniform(0.25, 1.0, (T, 1)).astype(np.float32)
    got, dbg = run_layer(w, torch, dev=dev, route_idx=idx, route_gate=gate)
    check_permutation(idx, dbg, w.E)
    assert list(dbg["counts"]) == counts
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, gate.astype(np.float64))
    err, eerr = normwise_err(got, ref), elementwise_err(got, ref)
    print(f"tile-group remainders: normwise {err:.3e}, elementwise {eerr:.3e}")
    assert err <= TOL["bf16"]
    assert np.all(np.isfinite(got))


def test_routing_override_single_expert_k1():
    T = 150
    w = synthetic.make("decode", T=T, d=256, f=512, k=1, seed=8)
    idx = np.full((T, 1), 5, np.int32)
    gate = np.ones((T, 1), np.float32)
    got, dbg = run_layer(w, torch, route_idx=idx, route_gate=gate)
    check_permutation(idx, dbg, w.E)
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, gate.astype(np.float64))
    assert normwise_err(got, ref) <= TOL["bf16"]


def test_zero_router_tie_break_and_gates():
    # all logits equal: experts (0, 1), gates exactly 1/8 (no renormalisation)
    w = synthetic.make("decode", T=40, d=256, f=256, seed=9)
    w.router_w[:] = 0
    got, dbg = run_layer(w, torch)
    assert np.all(dbg["idx"] == [0, 1])
    assert np.all(dbg["gate"] == np.float32(0.125))
    assert list(dbg["counts"]) == [40, 40, 0, 0, 0, 0, 0, 0]


def test_deterministic_bitwise():
    for T in (8, 300):
        w = synthetic.make("decode", T=T, d=256, f=512, seed=11)
        dev = dev_workload(w, torch)
        a, da = run_layer(w, torch, dev=dev)
        b, db = run_layer(w, torch, dev=dev)
        np.testing.assert_array_equal(a, b)
        for n in da:
            np.testing.assert_array_equal(da[n], db[n])


def test_power_of_two_scaling_exact():
    # doubling the down weights doubles the output exactly (bf16 * 2 is exact, fp32 sums scale exactly)
    w = synthetic.make("decode", T=50, d=256, f=512, seed=12)
    a, _ = run_layer(w, torch)
    w2 = synthetic.make("decode", T=50, d=256, f=512, seed=12)
    w2.w_down = synthetic.f32_to_bf16_bits(2 * synthetic.bf16_bits_to_f32(w2.w_down))
    b, _ = run_layer(w2, torch)
    np.testing.assert_array_equal(b, 2 * a)


def test_zero_tokens_noop():
    w = synthetic.make("decode", T=4, d=256, f=256)
    dev = dev_workload(w, torch)
    x0 = dev["x"][:0]
    out = torch.full((0, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    gm.grok_moe_forward(x0, dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], out=out)
    torch.cuda.synchronize()


def test_plain_entry_points_match_ex():
    w = synthetic.make("decode", T=20, d=256, f=512, seed=13)
    dev = dev_workload(w, torch)
    ref, _ = gm.grok_moe_forward_ex(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"])
    out = gm.grok_moe_forward(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    w8 = synthetic.make("int8", T=20, d=256, f=512, seed=13)
    d8 = dev_workload(w8, torch)
    r8, _ = gm.grok_moe_forward_ex(d8["x"], d8["router_w"], d8["w_gate"], d8["w_up"], d8["w_down"],
                                   scales=d8["scales"])
    o8 = gm.grok_moe_forward_w8(d8["x"], d8["router_w"], d8["w_gate"], d8["w_up"], d8["w_down"], d8["scales"])
    wf = synthetic.make("tiny_f32", T=20, seed=13)
    df = dev_workload(wf, torch)
    rf, _ = gm.grok_moe_forward_ex(df["x"], df["router_w"], df["w_gate"], df["w_up"], df["w_down"])
    of = gm.grok_moe_forward_f32(df["x"], df["router_w"], df["w_gate"], df["w_up"], df["w_down"])
    torch.cuda.synchronize()
    assert torch.equal(o8, r8) and torch.equal(of, rf)


def test_binding_errors_raise():
    w = synthetic.make("decode", T=4, d=256, f=256)
    dev = dev_workload(w, torch)
    with pytest.raises(gm.GrokMoeError) as ei:
        gm.grok_moe_forward(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], k=9)
    assert ei.value.code == gm.EINVAL
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gm.GrokMoeError) as ei:
        gm.grok_moe_forward_ex(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], workspace=ws)
    assert ei.value.code == gm.EWORKSPACE
    # sizes the library cannot check are checked by the binding before any launch: a wrong-shape out
    # and wrong-length 8-bit scales raise, and the out buffer is left untouched
    out = torch.full((w.T, w.d + 64), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gm.grok_moe_forward(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], out=out)
    with pytest.raises(ValueError):
        gm.grok_moe_forward_ex(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], out=out)
    w8 = synthetic.make("int8", T=4, d=256, f=256)
    d8 = dev_workload(w8, torch)
    short = d8["scales"][:-1].contiguous()
    with pytest.raises(ValueError):
        gm.grok_moe_forward_w8(d8["x"], d8["router_w"], d8["w_gate"], d8["w_up"], d8["w_down"], short)
    with pytest.raises(ValueError):
        gm.grok_moe_forward_ex(d8["x"], d8["router_w"], d8["w_gate"], d8["w_up"], d8["w_down"], scales=short)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


@pytest.mark.parametrize("T", [40, 2049])
def test_router_sends_every_token_to_two_experts(T):
    # a constant feature with router weights +100 (expert 0) and +50 (expert 5): every token picks
    # (0, 5), so two segments hold all T rows and six experts are empty (bf16-exact inputs)
    w = synthetic.make("decode", T=T, d=256, f=512, seed=14)
    w.x[:, w.d - 1] = synthetic.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    bias = np.zeros(w.E, np.float32)
    bias[0], bias[5] = 100.0, 50.0
    w.router_w[:, w.d - 1] = synthetic.f32_to_bf16_bits(bias)
    got, dbg, _ = _full_check(w)
    assert (dbg["idx"] == [0, 5]).all()
    assert list(dbg["counts"]) == [T, 0, 0, 0, 0, T, 0, 0]


@pytest.mark.parametrize("E,k,cf", [(8, 2, 0.0), (256, 8, 0.0), (8, 2, 0.9), (256, 8, 1.1)])
def test_permutation_many_blocks(E, k, cf):
    # 70,000 tokens: more than 256 sub-chunks of 256 tokens, so each permutation block walks two
    # sub-chunks (the last one ragged). Caller routing with skewed expert popularity (weighted
    # sampling of k distinct experts per token); permutation bit-exact against the oracle's, with
    # and without a capacity cap; outputs checked on a sample of tokens
    T = 70000
    w = synthetic.make("decode", T=T, d=256, f=256, E=E, k=k, seed=E + k, capacity_factor=cf)
    rng = np.random.default_rng(E * 31 + k)
    weight = 1.0 / (1.0 + np.arange(E)) ** 0.7
    keys = np.log(rng.random((T, E))) / weight                 # top-k keys: sampling without replacement
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    gate = rng.random((T, k)).astype(np.float32)
    got, dbg = run_layer(w, torch, route_idx=idx, route_gate=gate)
    cap = oracle.capacity(cf, T, E, k)
    c, o, p, pos = oracle.permute_cap(idx, E, cap)
    np.testing.assert_array_equal(dbg["counts"], c)
    np.testing.assert_array_equal(dbg["offsets"], o)
    np.testing.assert_array_equal(dbg["perm"][:o[-1]], p[:o[-1]])
    np.testing.assert_array_equal(dbg["pos"], pos)
    if cf > 0:
        assert c.max() == cap and (pos < 0).any()
    toks = np.sort(rng.choice(T, 256, replace=False))
    # dropped assignments contribute nothing: gate 0 in the oracle
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx,
                                       np.where(pos >= 0, gate, 0.0).astype(np.float64), tokens=toks)
    assert normwise_err(got[toks], ref) <= TOL["bf16"]


@pytest.mark.parametrize("w_dtype,T,sizes", [("bf16", 1100, [0, 1, 319, 320, 321, 640, 599, 0]),
                                              ("bf16", 1100, [0, 255, 256, 257, 512, 513, 1, 406]),
                                              ("bf16", 2100, [0, 255, 256, 257, 1024, 1025, 1, 1382]),
                                              ("i8", 1100, [0, 1, 319, 320, 321, 640, 599, 0]),
                                              ("i8", 2100, [0, 255, 256, 257, 1024, 1025, 1, 1382]),
                                              ("i8", 228, [1, 17, 33, 49, 65, 81, 97, 113]),
                                              ("i8", 64, [1, 17, 33, 49, 28, 0, 0, 0])])
def test_tile_boundaries_and_empty_experts(w_dtype, T, sizes):
    # 1,100 tokens at top-2 average 275 rows per expert, so bf16 weights run 320-row tiles (8-bit: 128-row);
    # 2,100 tokens average 525, the same tiles (8-bit: tiled, 256-row). Segments of 0, 1, 255 .. 257,
    # 319 .. 321, 512, 513, 640, 1024 and 1025 rows put tile edges on both sides of every boundary, and
    # empty first and last experts must be skipped by the tile table. With 8-bit weights and 65 .. 256
    # (up to 64) tokens the streaming kernel runs 128-row (64-row) chunks, and segments of 1, 17, .., 113
    # rows take every count of 16-row MFMA tiles it computes (1 .. 8, or 1 .. 4)
    E, k = 8, 2
    assert sum(sizes) == T * k
    labels = np.repeat(np.arange(E, dtype=np.int32), sizes)            # sorted by expert, 2T long
    idx = np.stack([labels[:T], labels[T:]], axis=1)                   # runs < T long: distinct per token
    assert np.all(idx[:, 0] != idx[:, 1])
    rng = np.random.default_rng(11)
    idx = idx[rng.permutation(T)]
    gate = rng.random((T, k)).astype(np.float32)
    w = synthetic.make("decode", T=T, d=256, f=512, E=E, k=k, seed=12, w_dtype=w_dtype)
    got, dbg = run_layer(w, torch, route_idx=idx, route_gate=gate)
    check_permutation(idx, dbg, E)
    assert list(dbg["counts"]) == sizes
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, gate.astype(np.float64),
                                       scales=w.scales)
    assert normwise_err(got, ref) <= TOL["i8" if w_dtype == "i8" else "bf16"]


@pytest.mark.parametrize("E,k,ns", [(8, 2, 0), (72, 8, 1)])
def test_non_finite_tokens_stay_local(E, k, ns):
    # inputs outside the contract (NaN / Inf in some tokens) must not crash, hang or leak into other
    # tokens: every GEMM row, router row and combine row is computed from its own token only
    T = 100
    w = synthetic.make("dsv3_decode" if ns else "decode", T=T, d=256, f=256, E=E, k=k, seed=21)
    bad = [5, 17, 63]
    nan_bits, inf_bits = np.uint16(0x7FC0), np.uint16(0x7F80)
    w.x = w.x.copy()
    w.x[5, :] = nan_bits
    w.x[17, 3] = inf_bits
    w.x[63, 200] = nan_bits
    got, dbg = run_layer(w, torch)
    clean = np.array([t for t in range(T) if t not in bad])
    ref = oracle.layer(w.x[clean], w.router_w, w.w_gate, w.w_up, w.w_down, w.k,
                       activation=oracle.SILU if w.activation == "silu" else oracle.GELU,
                       renormalize=w.renormalize, n_shared=w.n_shared, router_bias=w.router_bias)
    np.testing.assert_array_equal(dbg["idx"][clean], ref["idx"])
    assert np.all(np.isfinite(got[clean]))
    assert normwise_err(got[clean], ref["out"]) <= TOL["bf16"]
    # the routing of the bad tokens is valid or dropped (-1), never outside [0, E + ns)
    assert np.all((dbg["idx"][bad] >= -1) & (dbg["idx"][bad] < E + ns))


@pytest.mark.parametrize("T,d,f,w_dtype", [
    (5, 320, 384, "bf16"),       # weight streaming; the down pass's last 128-channel workgroup is half past d
    (40, 448, 384, "bf16"),
    (24, 320, 384, "i8"),        # 8-bit weights with d % 128 != 0 take the tiled path even at small T
    (200, 320, 384, "i8"),
    (200, 320, 384, "bf16"),     # tiled, 128-row tiles; the down pass's 256-channel tile is ragged
    (700, 448, 1408, "bf16"),    # tiled, 256-row tiles
    (2100, 320, 384, "bf16"),    # ping-pong tiles (525 rows per expert: a full and a partial tile)
    (1200, 320, 384, "bf16"),    # 320-row ping-pong tiles (300 rows per expert); ragged down tile
    (8, 6208, 1408, "bf16"),     # d = 97 x 64, f = 11 x 128
    (8, 6208, 1408, "i8"),
    (2100, 6208, 1408, "bf16"),
    (1200, 6208, 1408, "bf16"),  # 320-row ping-pong tiles, two down splits
    (2100, 384, 1408, "i8"),     # 8-bit at 525 rows per expert: tiled 256-row tiles, the down pass's last tile half past d
])
def test_widths_multiple_of_64_and_128(T, d, f, w_dtype):
    # the boundary takes d % 64 == 0 and f % 128 == 0: every kernel family runs ragged last channel tiles
    # of the down projection (output channels past d are computed from clamped weight rows and not stored)
    w = synthetic.make("decode", T=T, d=d, f=f, seed=T + d + f, w_dtype=w_dtype)
    if w_dtype == "i8":
        w.scales = synthetic.random_scales(w.E, w.d, w.f, seed=d)
    got, dbg = run_layer(w, torch)
    probs, oidx, _ = oracle.route(w.x, w.router_w, w.k)
    check_routing(dbg["idx"], dbg["gate"], probs)
    check_permutation(dbg["idx"], dbg, w.E)
    gates = np.take_along_axis(probs, dbg["idx"].astype(np.int64), 1)
    toks = None
    if T * d * f > 2e9:   # sample: both edges of every 256- and 320-row tile of every expert, 24 random tokens
        offs, perm = dbg["offsets"], dbg["perm"]
        pick = set(np.random.default_rng(T).choice(T, 24, replace=False).tolist())
        for e in range(w.E):
            n = int(offs[e + 1] - offs[e])
            for bm in (256, 320):
                for m0 in range(0, n, bm):
                    pick.update((int(perm[offs[e] + m0]), int(perm[offs[e] + min(n, m0 + bm) - 1])))
        toks = sorted(pick)
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, dbg["idx"], gates, scales=w.scales,
                                       tokens=toks)
    sub = got if toks is None else got[toks]
    err = normwise_err(sub, ref)
    tol = TOL["i8" if w_dtype == "i8" else "bf16"]
    print(f"[widths] T={T} d={d} f={f} {w_dtype}: {len(sub)} tokens, normwise error {err:.3e}", flush=True)
    assert err <= tol and np.all(np.isfinite(got))
