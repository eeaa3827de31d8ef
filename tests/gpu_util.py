"""Shared helpers of the GPU parity tests: device copies of workloads, one layer call
through the C ABI with debug outputs, and the comparison rules."""
from __future__ import annotations

import numpy as np

import mixture_experts_transformer_gemm_amd as gm
import oracle
import synthetic

TOL = {"bf16": 2e-2, "i8": 5e-2, "f32": 1e-4}   # per-token normwise relative error
TIE_WINDOW = 1e-6                                # routing: probability window for near-ties


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_workload(w: synthetic.Workload, torch):
    return {n: to_dev(getattr(w, n), torch)
            for n in ("x", "router_w", "w_gate", "w_up", "w_down", "scales", "norm_pre", "norm_post", "router_bias")}


def run_layer(w: synthetic.Workload, torch, dev=None, route_idx=None, route_gate=None, debug=True):
    """One layer call via grok_moe_forward_ex, with the workload's variant knobs.
    Returns (out f64 [T,d], dbg numpy dict; bf16 tensors as uint16 bits)."""
    dev = dev or dev_workload(w, torch)
    ri = None if route_idx is None else torch.from_numpy(np.ascontiguousarray(route_idx, np.int32)).cuda()
    rg = None if route_gate is None else torch.from_numpy(np.ascontiguousarray(route_gate, np.float32)).cuda()
    out, dbg = gm.grok_moe_forward_ex(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"],
                                      k=w.k, scales=dev["scales"], route_idx=ri, route_gate=rg, debug=debug,
                                      activation=gm.ACT_SILU if w.activation == "silu" else gm.ACT_GELU,
                                      renormalize=w.renormalize, capacity_factor=w.capacity_factor,
                                      norm_pre=dev["norm_pre"], norm_post=dev["norm_post"], norm_eps=w.norm_eps,
                                      n_shared=w.n_shared, router_bias=dev["router_bias"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    host = {}
    for n, t in dbg.items():
        host[n] = t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()
    return got, host


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over tokens of ||got_t - ref_t||_inf / ||ref_t||_inf."""
    if got.size == 0:
        return 0.0
    den = np.abs(ref).max(1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref).max(1) / den))


def elementwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over elements of |got - ref| / max(|ref|, 1e-3 * ||ref_t||_inf): the elementwise relative error,
    with entries near zero measured against a thousandth of their token's largest value."""
    if got.size == 0:
        return 0.0
    floor = 1e-3 * np.abs(ref).max(1, keepdims=True)
    den = np.maximum(np.abs(ref), floor)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den))


def check_routing(gidx: np.ndarray, ggate: np.ndarray, probs: np.ndarray):
    """GPU routing vs oracle probabilities: at each rank the chosen expert's oracle probability is
    within TIE_WINDOW of the oracle's rank-j probability, indices are distinct, and the GPU gate
    equals the oracle probability of its expert (fp32 rounding). Returns #tokens whose indices
    differ from the oracle's exact choice (legitimate only at near-ties)."""
    T, k = gidx.shape
    assert np.all((gidx >= 0) & (gidx < probs.shape[1]))
    srt = -np.sort(-probs, axis=1)[:, :k]
    chosen = np.take_along_axis(probs, gidx.astype(np.int64), 1)
    assert np.all(np.abs(chosen - srt) <= TIE_WINDOW), np.argwhere(np.abs(chosen - srt) > TIE_WINDOW)[:5]
    for j in range(k):
        for q in range(j):
            assert np.all(gidx[:, j] != gidx[:, q])
    assert np.all(np.abs(ggate.astype(np.float64) - chosen) <= 1e-6 * np.maximum(chosen, 1e-30) + 1e-12)
    return chosen


def check_permutation(gidx, dbg, E):
    """Bit-exact against the oracle's permutation of the GPU's own routing."""
    c, o, p, pos = oracle.permute(gidx, E)
    np.testing.assert_array_equal(dbg["counts"], c)
    np.testing.assert_array_equal(dbg["offsets"], o)
    np.testing.assert_array_equal(dbg["perm"], p)
    np.testing.assert_array_equal(dbg["pos"], pos)
