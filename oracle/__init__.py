"""CPU oracle for the Grok-1 MoE feed-forward layer (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the bench's CPU-baseline leg use this
package. The GPU library never imports, links or calls it, and the two share
no code: the only thing both sides consume is the seeded input data made by
the ``synthetic`` package.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, one
token and one expert at a time); this module only marshals numpy arrays. See
the header of ``moe_oracle.c`` for the definition it follows and the passages
of the pages it cites.

Parity pins: routing, permutation, GELU, the expert FFN, the whole layer and
the 8-bit scale indexing are each pinned by CPU tests (closed forms,
invariants, brute force, textbook special cases and independent library
routines), and so are the variants (``layer``: SiLU experts, renormalised
gates, capacity-factor drops, the sandwich sub-layer's RMSNorms and its bf16
rounding of the pre-norm) in ``tests/test_oracle_variants.py``. No function
here is left unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_handle = None

F64, F32, BF16, I8 = 0, 1, 2, 3
GELU, SILU = 0, 1


class _Layer(ctypes.Structure):
    # mirrors orc_layer in moe_oracle.c
    _fields_ = [("x", ctypes.c_void_p), ("xdt", ctypes.c_int), ("router_w", ctypes.c_void_p), ("rdt", ctypes.c_int),
                ("wg", ctypes.c_void_p), ("wu", ctypes.c_void_p), ("wd", ctypes.c_void_p), ("wdt", ctypes.c_int),
                ("scales", ctypes.c_void_p), ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64),
                ("E", ctypes.c_int), ("k", ctypes.c_int), ("act", ctypes.c_int), ("renormalize", ctypes.c_int),
                ("capacity_factor", ctypes.c_double), ("norm_pre", ctypes.c_void_p),
                ("norm_post", ctypes.c_void_p), ("norm_dt", ctypes.c_int), ("norm_eps", ctypes.c_double),
                ("n_shared", ctypes.c_int), ("router_bias", ctypes.c_void_p)]


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _handle
    if _handle is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_route.argtypes = [vp, ci, vp, ci, i64, i64, ci, ci, vp, vp, vp, ci]
        lib.oracle_permute.argtypes = [vp, i64, ci, ci, vp, vp, vp, vp]
        lib.oracle_expert.argtypes = [vp, ci, i64, vp, vp, vp, ci, vp, i64, i64, ci, ci, vp]
        lib.oracle_forward_given_routing.argtypes = [vp, ci, vp, vp, vp, ci, vp, vp, vp, i64, i64, i64, ci, ci,
                                                     vp, i64, vp, ci]
        lib.oracle_forward.argtypes = [vp, ci, vp, ci, vp, vp, vp, ci, vp, i64, i64, i64, ci, ci, vp, vp, vp, ci]
        lib.oracle_dense_onehot.argtypes = [vp, ci, vp, ci, vp, vp, vp, ci, vp, i64, i64, i64, ci, ci, vp, ci]
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_capacity.argtypes = [ctypes.c_double, i64, ci, ci]
        lib.oracle_capacity.restype = i64
        lib.oracle_route_v.argtypes = [vp, ci, vp, ci, i64, i64, ci, ci, ci, vp, vp, vp, vp, ci]
        lib.oracle_permute_cap.argtypes = [vp, i64, ci, ci, i64, ci, vp, vp, vp, vp]
        lib.oracle_rmsnorm.argtypes = [vp, ci, i64, i64, vp, ci, ctypes.c_double, vp]
        lib.oracle_layer.argtypes = [ctypes.POINTER(_Layer), vp, i64, vp, vp, vp, vp, vp, ci]
        for name in ("oracle_route", "oracle_permute", "oracle_expert", "oracle_forward_given_routing",
                     "oracle_forward", "oracle_dense_onehot", "oracle_route_v", "oracle_permute_cap",
                     "oracle_rmsnorm", "oracle_layer"):
            getattr(lib, name).restype = ci
        _handle = lib
    return _handle


def _dt(arr: np.ndarray, bf16: bool) -> int:
    if arr.dtype == np.float64:
        return F64
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16 and bf16:
        return BF16
    if arr.dtype == np.int8:
        return I8
    raise TypeError(f"unsupported oracle dtype {arr.dtype}")


def _c(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def gelu(z: float) -> float:
    return _lib().oracle_gelu(float(z))


def route(x: np.ndarray, router_w: np.ndarray, k: int, nthreads: int = 0
          ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns (probs [T,E] f64, idx [T,k] int32, gate [T,k] f64). uint16 arrays are bf16 bits."""
    x = np.ascontiguousarray(x)
    router_w = np.ascontiguousarray(router_w)
    T, d = x.shape
    E = router_w.shape[0]
    probs = np.zeros((T, E), np.float64)
    idx = np.zeros((T, k), np.int32)
    gate = np.zeros((T, k), np.float64)
    rc = _lib().oracle_route(x.ctypes.data, _dt(x, True), router_w.ctypes.data, _dt(router_w, True), T, d, E, k,
                             probs.ctypes.data, idx.ctypes.data, gate.ctypes.data, nthreads or threads())
    _check(rc, "route")
    return probs, idx, gate


def permute(idx: np.ndarray, E: int):
    """Returns (counts [E], offsets [E+1], perm [kT], pos [T,k]) as int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    pos = np.zeros((T, k), np.int32)
    rc = _lib().oracle_permute(idx.ctypes.data, T, E, k, counts.ctypes.data, offsets.ctypes.data,
                               perm.ctypes.data, pos.ctypes.data)
    _check(rc, "permute")
    return counts, offsets, perm, pos


def _wargs(w_gate, w_up, w_down, scales):
    w_gate = np.ascontiguousarray(w_gate)
    w_up = np.ascontiguousarray(w_up)
    w_down = np.ascontiguousarray(w_down)
    wdt = _dt(w_gate, True)
    if _dt(w_up, True) != wdt or _dt(w_down, True) != wdt:
        raise TypeError("gate/up/down weights must share one dtype")
    if wdt == I8:
        if scales is None:
            raise ValueError("8-bit weights need scales")
        scales = np.ascontiguousarray(scales, dtype=np.float32)
    else:
        scales = None
    return w_gate, w_up, w_down, wdt, scales


def expert(x: np.ndarray, t: int, e: int, w_gate, w_up, w_down, scales=None) -> np.ndarray:
    """Output of expert e alone for token t (d values, f64)."""
    x = np.ascontiguousarray(x)
    w_gate, w_up, w_down, wdt, scales = _wargs(w_gate, w_up, w_down, scales)
    E, f, d = w_gate.shape
    y = np.zeros(d, np.float64)
    rc = _lib().oracle_expert(x.ctypes.data, _dt(x, True), t, w_gate.ctypes.data, w_up.ctypes.data,
                              w_down.ctypes.data, wdt, _c(scales), d, f, E, e, y.ctypes.data)
    _check(rc, "expert")
    return y


def forward_given_routing(x, w_gate, w_up, w_down, idx, gate, scales=None,
                          tokens: Optional[Sequence[int]] = None, nthreads: int = 0) -> np.ndarray:
    """Steps 4-5 given routing. Returns [len(tokens) or T, d] f64."""
    x = np.ascontiguousarray(x)
    w_gate, w_up, w_down, wdt, scales = _wargs(w_gate, w_up, w_down, scales)
    E, f, d = w_gate.shape
    T = x.shape[0]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    k = idx.shape[1]
    tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    ntok = T if tok is None else tok.shape[0]
    out = np.zeros((ntok, d), np.float64)
    rc = _lib().oracle_forward_given_routing(x.ctypes.data, _dt(x, True), w_gate.ctypes.data, w_up.ctypes.data,
                                             w_down.ctypes.data, wdt, _c(scales), idx.ctypes.data,
                                             gate.ctypes.data, T, d, f, E, k, _c(tok), ntok, out.ctypes.data,
                                             nthreads or threads())
    _check(rc, "forward_given_routing")
    return out


def forward(x, router_w, w_gate, w_up, w_down, k: int, scales=None, nthreads: int = 0):
    """The whole layer. Returns (out [T,d] f64, idx [T,k] int32, gate [T,k] f64)."""
    x = np.ascontiguousarray(x)
    router_w = np.ascontiguousarray(router_w)
    w_gate, w_up, w_down, wdt, scales = _wargs(w_gate, w_up, w_down, scales)
    E, f, d = w_gate.shape
    T = x.shape[0]
    out = np.zeros((T, d), np.float64)
    idx = np.zeros((T, k), np.int32)
    gate = np.zeros((T, k), np.float64)
    rc = _lib().oracle_forward(x.ctypes.data, _dt(x, True), router_w.ctypes.data, _dt(router_w, True),
                               w_gate.ctypes.data, w_up.ctypes.data, w_down.ctypes.data, wdt, _c(scales), T, d, f,
                               E, k, out.ctypes.data, idx.ctypes.data, gate.ctypes.data, nthreads or threads())
    _check(rc, "forward")
    return out, idx, gate


def dense_onehot(x, router_w, w_gate, w_up, w_down, k: int, scales=None, nthreads: int = 0) -> np.ndarray:
    """Brute force: every expert on every token, one-hot(top-k) * gate mask."""
    x = np.ascontiguousarray(x)
    router_w = np.ascontiguousarray(router_w)
    w_gate, w_up, w_down, wdt, scales = _wargs(w_gate, w_up, w_down, scales)
    E, f, d = w_gate.shape
    T = x.shape[0]
    out = np.zeros((T, d), np.float64)
    rc = _lib().oracle_dense_onehot(x.ctypes.data, _dt(x, True), router_w.ctypes.data, _dt(router_w, True),
                                    w_gate.ctypes.data, w_up.ctypes.data, w_down.ctypes.data, wdt, _c(scales),
                                    T, d, f, E, k, out.ctypes.data, nthreads or threads())
    _check(rc, "dense_onehot")
    return out


# ---------------------------------------------------------------- variants
def silu(z: float) -> float:
    return _lib().oracle_silu(float(z))


def bf16_rne(v: float) -> int:
    """Bit pattern of the bf16 value nearest to v (ties to even)."""
    return int(_lib().oracle_bf16_rne(float(v)))


def capacity(c: float, T: int, E: int, k: int) -> int:
    """Rows each expert keeps under capacity factor c (-1: no cap, c <= 0)."""
    return int(_lib().oracle_capacity(float(c), T, E, k))


def route_v(x: np.ndarray, router_w: np.ndarray, k: int, renormalize: bool = False, bias=None,
            nthreads: int = 0):
    """route() with the optional selection bias (E fp32 values added to p for the top-k choice only)
    and the optional renormalisation of the k gates."""
    x = np.ascontiguousarray(x)
    router_w = np.ascontiguousarray(router_w)
    T, d = x.shape
    E = router_w.shape[0]
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (E,)
    probs = np.zeros((T, E), np.float64)
    idx = np.zeros((T, k), np.int32)
    gate = np.zeros((T, k), np.float64)
    rc = _lib().oracle_route_v(x.ctypes.data, _dt(x, True), router_w.ctypes.data, _dt(router_w, True), T, d, E, k,
                               int(bool(renormalize)), _c(bias), probs.ctypes.data, idx.ctypes.data,
                               gate.ctypes.data, nthreads or threads())
    _check(rc, "route_v")
    return probs, idx, gate


def permute_cap(idx: np.ndarray, E: int, cap: int, E_cap: Optional[int] = None):
    """permute() with at most `cap` rows per expert e < E_cap (default all; cap < 0: none). Dropped
    assignments get pos = -1; perm holds offsets[E] valid rows (the rest of the array is zero)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    pos = np.zeros((T, k), np.int32)
    rc = _lib().oracle_permute_cap(idx.ctypes.data, T, E, k, int(cap), E if E_cap is None else int(E_cap),
                                   counts.ctypes.data, offsets.ctypes.data, perm.ctypes.data, pos.ctypes.data)
    _check(rc, "permute_cap")
    return counts, offsets, perm, pos


def rmsnorm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm in double. uint16 arrays are bf16 bits."""
    v = np.ascontiguousarray(v)
    g = np.ascontiguousarray(g)
    T, d = v.shape
    out = np.zeros((T, d), np.float64)
    rc = _lib().oracle_rmsnorm(v.ctypes.data, _dt(v, True), T, d, g.ctypes.data, _dt(g, True), float(eps),
                               out.ctypes.data)
    _check(rc, "rmsnorm")
    return out


def layer(x, router_w, w_gate, w_up, w_down, k: int, scales=None, activation: int = GELU,
          renormalize: bool = False, capacity_factor: float = 0.0, norm_pre=None, norm_post=None,
          norm_eps: float = 1e-5, n_shared: int = 0, router_bias=None, tokens: Optional[Sequence[int]] = None,
          nthreads: int = 0):
    """The layer with its variants. The weights hold E routed experts (router_w has E rows) followed by
    n_shared shared experts. Returns dict(out [ntok, d] f64, idx, gate, pos [T, k + n_shared],
    u [T, d] or None)."""
    x = np.ascontiguousarray(x)
    router_w = np.ascontiguousarray(router_w)
    w_gate, w_up, w_down, wdt, scales = _wargs(w_gate, w_up, w_down, scales)
    Et, f, d = w_gate.shape
    E = router_w.shape[0]
    if Et != E + n_shared:
        raise ValueError(f"weights hold {Et} experts, router {E} + {n_shared} shared")
    T = x.shape[0]
    if router_bias is not None:
        router_bias = np.ascontiguousarray(router_bias, dtype=np.float32)
        assert router_bias.shape == (E,)
    L = _Layer()
    L.x, L.xdt = x.ctypes.data, _dt(x, True)
    L.router_w, L.rdt = router_w.ctypes.data, _dt(router_w, True)
    L.wg, L.wu, L.wd, L.wdt, L.scales = w_gate.ctypes.data, w_up.ctypes.data, w_down.ctypes.data, wdt, _c(scales)
    L.T, L.d, L.f, L.E, L.k = T, d, f, E, k
    L.act, L.renormalize, L.capacity_factor = int(activation), int(bool(renormalize)), float(capacity_factor)
    u = None
    if norm_pre is not None or norm_post is not None:
        norm_pre = np.ascontiguousarray(norm_pre)
        norm_post = np.ascontiguousarray(norm_post)
        if norm_pre.dtype != norm_post.dtype:
            raise TypeError("norm_pre and norm_post must share one dtype")
        L.norm_pre, L.norm_post, L.norm_dt = norm_pre.ctypes.data, norm_post.ctypes.data, _dt(norm_pre, True)
        u = np.zeros_like(x)
    L.norm_eps = float(norm_eps)
    L.n_shared, L.router_bias = int(n_shared), _c(router_bias)
    tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    ntok = T if tok is None else tok.shape[0]
    K = k + n_shared
    out = np.zeros((ntok, d), np.float64)
    idx = np.zeros((T, K), np.int32)
    gate = np.zeros((T, K), np.float64)
    pos = np.zeros((T, K), np.int32)
    rc = _lib().oracle_layer(ctypes.byref(L), _c(tok), ntok, out.ctypes.data, idx.ctypes.data, gate.ctypes.data,
                             pos.ctypes.data, _c(u), nthreads or threads())
    _check(rc, "layer")
    return dict(out=out, idx=idx, gate=gate, pos=pos, u=u)
