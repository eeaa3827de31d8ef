"""GPU parity at the Grok-1 layer's full sizes (d=6144, f=32768, E=8, k=2), in the
launch configuration the bench times (grok_moe_forward_ex with a caller workspace).

All tokens are checked for routing and permutation; outputs are compared with
the oracle on every token for the decode workloads and, for the larger ones, on
a seeded sample: the first and last row of every row tile the tiled kernels run
(every expert segment cut into tiles of the tile height the library picks for
that workload) and random tokens. Both the
per-token normwise error (the tolerance) and the elementwise error with a floor
of a thousandth of the token's largest value are computed and printed.
"""
import ctypes
import gc

import numpy as np
import pytest

import mixture_experts_transformer_gemm_amd as gm
import oracle
import synthetic
from gpu_util import TOL, check_permutation, check_routing, elementwise_err, normwise_err, run_layer

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _tile_rows(count, bm):
    """Rows (within a segment of `count` rows) at the edges of each bm-row tile."""
    rows = set()
    for m0 in range(0, count, bm):
        rows.update((m0, min(count, m0 + bm) - 1))
    return rows


def _sample_tokens(dbg, E, n_random, seed, bm=None):
    """Tokens whose rows sit at the first and last row of every bm-row tile of every expert segment (bm None:
    the segment edges only), plus n_random seeded tokens."""
    offs, perm = dbg["offsets"], dbg["perm"]
    pick = []
    for e in range(E):
        n = int(offs[e + 1] - offs[e])
        if n == 0:
            continue
        rows = {0, n - 1} if bm is None else _tile_rows(n, bm)
        pick += [int(perm[offs[e] + r]) for r in sorted(rows)]
    T = dbg["idx"].shape[0]
    pick += list(np.random.default_rng(seed).choice(T, size=min(n_random, T), replace=False))
    return sorted(set(pick))


def _tile_height(w):
    """Row-tile height the library runs for this workload's shape (grok_moe_tile_rows)."""
    a = gm.Args()
    a.T, a.d, a.f, a.E, a.k, a.n_shared = w.T, w.d, w.f, w.E, w.k, w.n_shared
    a.act_dtype = gm.F32 if w.act_dtype == "f32" else gm.BF16
    a.w_dtype = {"bf16": gm.BF16, "i8": gm.I8, "f32": gm.F32}[w.w_dtype]
    bm = gm.lib().grok_moe_tile_rows(ctypes.byref(a))
    assert bm > 0
    return bm


def _run_and_check(name, n_random=8, T=None, tiles=True):
    print(f"[fullsize] generating workload {name} (T={T or 'default'})", flush=True)
    w = synthetic.make(name, T=T)
    print(f"[fullsize] {name}: T={w.T} d={w.d} f={w.f} E={w.E} k={w.k} weights={w.w_dtype}", flush=True)
    got, dbg = run_layer(w, torch)
    probs, oidx, _ = oracle.route(w.x, w.router_w, w.k)
    check_routing(dbg["idx"], dbg["gate"], probs)
    mismatched = int(np.sum(np.any(dbg["idx"] != oidx, axis=1)))
    assert mismatched == 0, f"{mismatched} tokens routed differently from the oracle"
    check_permutation(dbg["idx"], dbg, w.E)
    assert np.all(np.isfinite(got))
    gates = np.take_along_axis(probs, dbg["idx"].astype(np.int64), 1)
    tokens = None if w.T <= 8 else _sample_tokens(dbg, w.E, n_random, seed=w.T, bm=_tile_height(w) if tiles else None)
    ref = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, dbg["idx"], gates, scales=w.scales,
                                       tokens=tokens)
    sub = got if tokens is None else got[tokens]
    err = normwise_err(sub, ref)
    ew = elementwise_err(sub, ref)
    tol = TOL["i8" if w.w_dtype == "i8" else "bf16"]
    print(f"[fullsize] {name}: {len(sub)} tokens checked, normwise error {err:.3e} (tol {tol}), elementwise "
          f"error {ew:.3e}", flush=True)
    assert err <= tol
    counts = dbg["counts"].copy()
    del w, got
    gc.collect()
    return dbg, counts


def test_decode_full():
    dbg, counts = _run_and_check("decode")
    assert counts.sum() == 16


def test_decode_T64_full():
    # 64-token decode: segments up to 64 rows in the weight-streaming kernel
    dbg, counts = _run_and_check("decode", n_random=8, T=64)
    assert counts.sum() == 128


def test_int8_decode_full():
    # 8-bit weights at decode size (weight streaming with int8 rows), every token checked
    dbg, counts = _run_and_check("int8", T=8)
    assert counts.sum() == 16


def test_int8_full():
    _run_and_check("int8", n_random=8)


def test_skew_full():
    dbg, counts = _run_and_check("skew", n_random=6)
    share = counts / counts.sum()
    assert share[0] > 0.4 and share[1] > 0.22


def test_int8_prefill_full():
    # 8-bit weights at the prefill size: the tiled 8-bit kernel (256-row tiles, int8 widened after the LDS read)
    dbg, counts = _run_and_check("int8", n_random=6, T=8192)
    assert counts.sum() == 2 * 8192


def test_prefill_full():
    dbg, counts = _run_and_check("prefill", n_random=6)
    pairs = {tuple(sorted(p)) for p in dbg["idx"].tolist()}
    assert len(pairs) == 28
    assert counts.sum() == 2 * 8192


def test_prefill_T32768_full():
    # four times the prefill batch: 65,536 rows, 26 row tiles of 320 per expert (53,248 gate/up
    # workgroups), and 4,992 down tiles (19.5 rounds of 256 CUs), so the down reduction runs in two
    # splits; every token's routing and the permutation are checked, outputs on a sample
    dbg, counts = _run_and_check("prefill", n_random=4, T=32768, tiles=False)
    assert counts.sum() == 2 * 32768
