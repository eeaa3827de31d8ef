"""GPU parity of the layer variants against the CPU oracle (``oracle.layer``):
SiLU experts with renormalised gates (the Mixtral variant), capacity-factor
drops, the sandwich sub-layer (RMSNorm before and after the MoE, plus the
residual) and the fine-grained layout (up to 256 routed experts, top-8, a
selection bias, shared experts), on the bf16, 8-bit and fp32 paths, small
shapes spanning the weight-streaming and tiled kernels, and at full Mixtral
8x22B / Grok-1 / DeepSeek-V3 sizes.

Rules as in the other parity tests: routing indices equal the oracle's; the
permutation (with dropped assignments at pos = -1) is bit-exact against the
oracle's capped permutation of the GPU routing; the pre-norm output u is
bit-exact against the oracle's bf16 rounding; outputs are within the per-token
normwise tolerance (2e-2 bf16, 5e-2 8-bit, 1e-4 fp32).
"""
import gc

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import TOL, TIE_WINDOW, dev_workload, normwise_err, run_layer

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _oracle(w, tokens=None):
    return oracle.layer(w.x, w.router_w, w.w_gate, w.w_up, w.w_down, w.k, scales=w.scales,
                        activation=oracle.SILU if w.activation == "silu" else oracle.GELU,
                        renormalize=w.renormalize, capacity_factor=w.capacity_factor, norm_pre=w.norm_pre,
                        norm_post=w.norm_post, norm_eps=w.norm_eps, n_shared=w.n_shared,
                        router_bias=w.router_bias, tokens=tokens)


def _tol(w):
    return TOL["f32" if w.act_dtype == "f32" else ("i8" if w.w_dtype == "i8" else "bf16")]


def _check(w, tokens=None, label=""):
    print(f"[variants] {label} T={w.T} d={w.d} f={w.f} E={w.E}+{w.n_shared} k={w.k} act={w.activation} "
          f"renorm={w.renormalize} cap={w.capacity_factor} sandwich={w.norm_pre is not None} "
          f"bias={w.router_bias is not None} w={w.w_dtype}", flush=True)
    got, dbg = run_layer(w, torch)
    ref = _oracle(w, tokens=tokens)
    if w.norm_pre is not None:
        np.testing.assert_array_equal(dbg["u"], ref["u"])          # pre-norm output, bit-exact
    np.testing.assert_array_equal(dbg["idx"], ref["idx"])          # routing decided on u, fp64 logits
    gate_tol = 1e-6 * np.maximum(ref["gate"], 1e-30) + 1e-12
    assert np.all(np.abs(dbg["gate"].astype(np.float64) - ref["gate"]) <= gate_tol)
    if w.renormalize:
        np.testing.assert_allclose(dbg["gate"][:, :w.k].sum(axis=1), 1.0, atol=1e-6)
    cap = oracle.capacity(w.capacity_factor, w.T, w.E, w.k)
    c, o, p, pos = oracle.permute_cap(dbg["idx"], w.E + w.n_shared, cap, E_cap=w.E)
    np.testing.assert_array_equal(dbg["counts"], c)
    np.testing.assert_array_equal(dbg["offsets"], o)
    np.testing.assert_array_equal(dbg["perm"][:o[-1]], p[:o[-1]])
    np.testing.assert_array_equal(dbg["pos"], pos)
    np.testing.assert_array_equal(dbg["pos"], ref["pos"])
    sub = got if tokens is None else got[tokens]
    err = normwise_err(sub, ref["out"])
    print(f"[variants] {label}: normwise error {err:.3e} (tol {_tol(w)})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= _tol(w), f"normwise error {err:.3e}"
    return got, dbg, ref


# ---------------------------------------------------------------- SiLU + renormalised gates (Mixtral)
@pytest.mark.parametrize("T", [1, 5, 64, 100, 300, 777])
def test_mixtral_variant_bf16(T):
    w = synthetic.make("mixtral_decode", T=T, d=256, f=512, seed=200 + T)
    _check(w, label="mixtral bf16")


@pytest.mark.parametrize("T", [40, 513])
def test_silu_int8(T):
    w = synthetic.make("int8", T=T, d=256, f=512, seed=T, activation="silu", renormalize=True)
    w.scales = synthetic.random_scales(w.E, w.d, w.f, seed=T)
    _check(w, label="silu int8")


def test_silu_f32():
    w = synthetic.make("tiny_f32", activation="silu", renormalize=True)
    _check(w, label="silu f32")


def test_renormalised_zero_router():
    w = synthetic.make("mixtral_decode", T=30, d=256, f=256, seed=3)
    w.router_w[:] = 0
    got, dbg, _ = _check(w, label="renorm zero router")
    assert np.all(dbg["idx"] == [0, 1]) and np.all(dbg["gate"] == np.float32(0.5))


# ---------------------------------------------------------------- capacity
@pytest.mark.parametrize("T,cf", [(40, 0.5), (64, 1.0), (300, 1.0), (777, 0.75), (1600, 1.25)])
def test_capacity_skewed_bf16(T, cf):
    w = synthetic.make("skew", T=T, d=256, f=512, seed=T, capacity_factor=cf)
    got, dbg, ref = _check(w, label="capacity")
    assert (dbg["pos"] == -1).any(), "the skewed routing must overflow"
    assert dbg["counts"].max() <= oracle.capacity(cf, T, w.E, w.k)


def test_capacity_int8():
    w = synthetic.make("skew", T=200, d=256, f=512, seed=5, w_dtype="i8", capacity_factor=0.8)
    _check(w, label="capacity int8")


def test_capacity_zero_rows_gives_zero_output():
    w = synthetic.make("decode", T=50, d=256, f=256, seed=6, capacity_factor=1e-3)
    got, dbg, _ = _check(w, label="capacity 0 rows")
    assert (dbg["pos"] == -1).all() and (dbg["counts"] == 0).all()
    assert (got == 0.0).all()


# ---------------------------------------------------------------- sandwich sub-layer
@pytest.mark.parametrize("T", [1, 8, 64, 300])
def test_sandwich_bf16(T):
    w = synthetic.make("decode", T=T, d=256, f=512, seed=300 + T, sandwich=True)
    _check(w, label="sandwich bf16")


def test_sandwich_f32_and_int8():
    _check(synthetic.make("tiny_f32", sandwich=True), label="sandwich f32")
    w = synthetic.make("int8", T=40, d=256, f=512, seed=4, sandwich=True)
    _check(w, label="sandwich int8")


def test_sandwich_zero_experts_is_the_residual():
    w = synthetic.make("decode", T=70, d=256, f=256, seed=7, sandwich=True)
    w.w_down = np.zeros_like(w.w_down)
    got, _, _ = _check(w, label="sandwich zero experts")
    np.testing.assert_array_equal(got, synthetic.bf16_bits_to_f32(w.x).astype(np.float64))


def test_all_variants_together():
    w = synthetic.make("skew", T=200, d=256, f=512, seed=8, activation="silu", renormalize=True,
                       capacity_factor=0.9, sandwich=True)
    got, dbg, _ = _check(w, label="all variants")
    dropped = np.all(dbg["pos"] == -1, axis=1)
    if dropped.any():   # tokens whose every assignment overflowed carry the residual only
        np.testing.assert_array_equal(got[dropped], synthetic.bf16_bits_to_f32(w.x[dropped]).astype(np.float64))


def test_variants_deterministic_bitwise():
    w = synthetic.make("skew", T=300, d=256, f=512, seed=9, activation="silu", renormalize=True,
                       capacity_factor=0.9, sandwich=True)
    dev = dev_workload(w, torch)
    a, da = run_layer(w, torch, dev=dev)
    b, db = run_layer(w, torch, dev=dev)
    np.testing.assert_array_equal(a, b)
    for n in da:
        np.testing.assert_array_equal(da[n], db[n])


# ---------------------------------------------------------------- full sizes
def _sample(dbg, E, T, n_random, seed):
    offs, perm = dbg["offsets"], dbg["perm"]
    pick = []
    for e in range(E):
        if offs[e + 1] > offs[e]:
            pick += [int(perm[offs[e]]), int(perm[offs[e + 1] - 1])]
    pick += list(np.random.default_rng(seed).choice(T, size=min(n_random, T), replace=False))
    return sorted(set(pick))


def test_mixtral_decode_full():
    # Mixtral 8x22B expert shapes (d=6144, f=16384), SiLU, renormalised gates, 8 tokens, all checked
    w = synthetic.make("mixtral_decode")
    _check(w, label="mixtral decode full")
    del w
    gc.collect()


def test_sandwich_decode_full():
    w = synthetic.make("decode", sandwich=True)
    _check(w, label="sandwich decode full")
    del w
    gc.collect()


def test_capacity_skew_full_sampled():
    # full Grok-1 shapes at the skewed 2048-token workload with capacity factor 1.0:
    # experts 0 and 1 overflow; routing/permutation for all tokens, outputs on a sample
    w = synthetic.make("skew", capacity_factor=1.0)
    got, dbg = run_layer(w, torch)
    ref_all = _oracle(w, tokens=[0])                 # routing + capped permutation of every token
    np.testing.assert_array_equal(dbg["idx"], ref_all["idx"])
    np.testing.assert_array_equal(dbg["pos"], ref_all["pos"])
    assert dbg["counts"][0] == oracle.capacity(1.0, w.T, w.E, w.k) == 512
    toks = _sample(dbg, w.E, w.T, 6, seed=1)
    dropped = [t for t in range(w.T) if (dbg["pos"][t] == -1).all()][:2]
    toks = sorted(set(toks + dropped))
    ref = _oracle(w, tokens=toks)
    err = normwise_err(got[toks], ref["out"])
    print(f"[variants] capacity skew full: {len(toks)} tokens, normwise error {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    del w
    gc.collect()


# ---------------------------------------------------------------- fine-grained: many experts, bias, shared experts
@pytest.mark.parametrize("T,E", [(1, 256), (8, 256), (64, 256), (300, 256), (1000, 256), (40, 72), (200, 100)])
def test_fine_grained_bf16(T, E):
    # E > 64: the split-K fp64 MFMA router GEMM + per-token top-k; top-8, one shared expert, selection bias
    w = synthetic.make("dsv3_decode", T=T, d=256, f=256, E=E, seed=400 + T)
    got, dbg, _ = _check(w, label="fine-grained")
    assert (dbg["idx"][:, 8] == E).all() and (dbg["gate"][:, 8] == 1.0).all()
    assert dbg["counts"][E] == T                      # the shared expert runs every token


def test_fine_grained_fused_router_two_shared():
    # E <= 64 keeps the one-kernel router; bias and two shared experts
    w = synthetic.make("dsv3_decode", T=90, d=256, f=256, E=32, k=4, n_shared=2, seed=5)
    _check(w, label="E=32 two shared")


@pytest.mark.parametrize("T", [4100, 2000])
def test_fine_grained_pingpong_shared(T):
    # T tokens over 32 routed experts (top-4) and one shared expert, SiLU epilogue, on the
    # ping-pong kernel. 4,100 tokens: about 621 rows per expert, and the shared expert's 4,100
    # rows make 13 row tiles of one expert (a group of 8 and a last group of 5, the last tile
    # 260 rows). 2,000 tokens: about 303 rows per expert (the shared expert: 7 row tiles, the
    # last of 80 rows)
    w = synthetic.make("dsv3_decode", T=T, d=256, f=256, E=32, k=4, seed=11)
    _, dbg, _ = _check(w, label="fine-grained ping-pong")
    assert dbg["counts"][32] == T


def test_fine_grained_int8_and_capacity():
    w = synthetic.make("dsv3_decode", T=120, d=256, f=256, seed=6, w_dtype="i8")
    w.scales = synthetic.random_scales(w.E + w.n_shared, w.d, w.f, seed=6)
    _check(w, label="fine-grained int8")
    w = synthetic.make("dsv3_decode", T=400, d=256, f=256, seed=7, capacity_factor=0.5, skew=True)
    got, dbg, _ = _check(w, label="fine-grained capacity")
    assert (dbg["pos"][:, :8] == -1).any() and (dbg["pos"][:, 8] >= 0).all()   # shared expert never capped


def test_fine_grained_split_gateup_with_capacity():
    # 48 tokens over 256 experts with d = f = 256: the streaming gate/up runs in two reduction
    # splits (fp32 sums + glu_splits_kernel), here with capped, skewed routing (drops) as well
    w = synthetic.make("dsv3_decode", T=48, d=256, f=256, seed=9, capacity_factor=0.5, skew=True)
    got, dbg, _ = _check(w, label="fine-grained split gate/up, capacity")
    assert (dbg["pos"][:, :8] == -1).any() and (dbg["pos"][:, 8] >= 0).all()


def test_fine_grained_routing_override():
    T, E = 50, 256
    # GELU experts: the oracle's forward_given_routing evaluates the GELU layer on a given routing
    w = synthetic.make("dsv3_decode", T=T, d=256, f=256, seed=8, activation="gelu")
    rng = np.random.default_rng(8)
    idx = np.stack([rng.choice(E, size=8, replace=False) for _ in range(T)]).astype(np.int32)
    gate = rng.uniform(0.01, 0.3, size=(T, 8)).astype(np.float32)
    idx[3, 2] = E          # the shared expert's index is not a routed expert: dropped
    idx[7, 0] = -5         # out of range: dropped
    got, dbg = run_layer(w, torch, route_idx=idx, route_gate=gate)
    dropped = (idx < 0) | (idx >= E)
    np.testing.assert_array_equal(dbg["idx"][:, :8], np.where(dropped, -1, idx))
    assert (dbg["pos"][:, :8][dropped] == -1).all() and (dbg["pos"][:, :8][~dropped] >= 0).all()
    assert (dbg["idx"][:, 8] == E).all() and (dbg["gate"][:, 8] == 1.0).all()
    ref_idx = np.where(dropped, 0, idx)                # any valid expert, with gate 0
    ref_gate = np.where(dropped, 0.0, gate.astype(np.float64))
    full_idx = np.concatenate([ref_idx, np.full((T, 1), E, np.int32)], axis=1)
    full_gate = np.concatenate([ref_gate, np.ones((T, 1))], axis=1)
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, full_idx, full_gate)
    assert normwise_err(got, ref) <= TOL["bf16"]


def test_dsv3_decode_full():
    # DeepSeek-V3 shapes: d=7168, 256 routed experts of width 2048, top-8, one shared expert, 8 tokens
    w = synthetic.make("dsv3_decode")
    _check(w, label="dsv3 decode full")
    del w
    gc.collect()


def test_dsv3_prefill_full_sampled():
    w = synthetic.make("dsv3_prefill")
    print(f"[variants] dsv3 prefill full: T={w.T}", flush=True)
    got, dbg = run_layer(w, torch)
    ref_all = _oracle(w, tokens=[0])
    np.testing.assert_array_equal(dbg["idx"], ref_all["idx"])
    c, o, p, pos = oracle.permute_cap(dbg["idx"], w.E + w.n_shared, -1)
    np.testing.assert_array_equal(dbg["counts"], c)
    np.testing.assert_array_equal(dbg["pos"], pos)
    cand = _sample(dbg, w.E + w.n_shared, w.T, 6, seed=2)
    toks = sorted(np.random.default_rng(3).choice(cand, size=min(40, len(cand)), replace=False).tolist())
    ref = _oracle(w, tokens=toks)
    err = normwise_err(got[toks], ref["out"])
    print(f"[variants] dsv3 prefill full: {len(toks)} tokens, normwise error {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    del w
    gc.collect()


def _full_sampled(w, label, n_random=6, max_tokens=40):
    print(f"[variants] {label}: T={w.T}", flush=True)
    got, dbg = run_layer(w, torch)
    ref_all = _oracle(w, tokens=[0])
    np.testing.assert_array_equal(dbg["idx"], ref_all["idx"])
    np.testing.assert_array_equal(dbg["pos"], ref_all["pos"])
    if w.norm_pre is not None:
        np.testing.assert_array_equal(dbg["u"], ref_all["u"])
    cand = _sample(dbg, w.E + w.n_shared, w.T, n_random, seed=4)
    toks = sorted(np.random.default_rng(5).choice(cand, size=min(max_tokens, len(cand)), replace=False).tolist())
    ref = _oracle(w, tokens=toks)
    err = normwise_err(got[toks], ref["out"])
    print(f"[variants] {label}: {len(toks)} tokens, normwise error {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_mixtral_prefill_full_sampled():
    # Mixtral 8x22B shapes at 8192 tokens: the tiled path with SiLU and renormalised gates
    w = synthetic.make("mixtral_prefill")
    _full_sampled(w, "mixtral prefill full")
    del w
    gc.collect()


def test_sandwich_prefill_full_sampled():
    # the sandwich sub-layer at the Grok-1 prefill shape (pre-norm output checked bitwise for all tokens)
    w = synthetic.make("prefill", sandwich=True)
    _full_sampled(w, "sandwich prefill full")
    del w
    gc.collect()
