"""Python binding of the MI355X Grok-1 MoE feed-forward library (libgrok_moe.so).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library; torch supplies device memory and the current stream. The names
mirror the C ABI in include/grok_moe.h, with the sizes taken from the tensor
shapes:

* ``grok_moe_forward``     bf16 activations and weights
* ``grok_moe_forward_w8``  bf16 activations, int8 weights + fp32 per-channel scales
* ``grok_moe_forward_f32`` fp32 everything
* ``grok_moe_forward_ex``  any of the above with caller workspace, optional
  routing override and debug outputs
* ``grok_moe_forward_static`` the ``_ex`` layer with the library's static
  per-device workspace (no allocation; shapes up to STATIC_WORKSPACE_BYTES)
* ``grok_moe_workspace_bytes``, ``grok_moe_status_string``

Layouts: x, out [T, d]; router_w [E, d]; w_gate, w_up [E, f, d]; w_down [E, d, f].
If the library is not built, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgrok_moe.so")

BF16, F32, I8 = 0, 1, 2
ACT_GELU, ACT_SILU = 0, 1
OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
STAGES = ("router", "permute", "gate_up", "down", "combine")

EXPORTED = ("grok_moe_workspace_bytes", "grok_moe_workspace_bytes_ex", "grok_moe_tile_rows", "grok_moe_forward_ex",
            "grok_moe_forward", "grok_moe_forward_w8", "grok_moe_forward_f32", "grok_moe_forward_static",
            "grok_moe_status_string")
STATIC_WORKSPACE_BYTES = 64 << 20   # GROK_MOE_STATIC_WORKSPACE_BYTES


class GrokMoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {grok_moe_status_string(code)} (status {code})")


class Args(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("router_w", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("route_idx", ctypes.c_void_p), ("route_gate", ctypes.c_void_p),
                ("activation", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("capacity_factor", ctypes.c_double),
                ("norm_pre", ctypes.c_void_p), ("norm_post", ctypes.c_void_p), ("norm_eps", ctypes.c_double),
                ("n_shared", ctypes.c_int32), ("router_bias", ctypes.c_void_p)]


class Debug(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("events", ctypes.c_void_p * 6), ("u", ctypes.c_void_p)]


_lib_handle = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               "g.build()'` (hipcc, gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        h.grok_moe_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32]
        h.grok_moe_workspace_bytes.restype = ctypes.c_size_t
        h.grok_moe_workspace_bytes_ex.argtypes = [ctypes.POINTER(Args)]
        h.grok_moe_workspace_bytes_ex.restype = ctypes.c_size_t
        h.grok_moe_tile_rows.argtypes = [ctypes.POINTER(Args)]
        h.grok_moe_tile_rows.restype = ctypes.c_int32
        h.grok_moe_forward_ex.argtypes = [ctypes.POINTER(Args), vp, ctypes.c_size_t, ctypes.POINTER(Debug), vp]
        h.grok_moe_forward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
        h.grok_moe_forward_w8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
        h.grok_moe_forward_f32.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
        h.grok_moe_forward_static.argtypes = [ctypes.POINTER(Args), ctypes.POINTER(Debug), vp]
        for n in ("grok_moe_forward_ex", "grok_moe_forward", "grok_moe_forward_w8", "grok_moe_forward_f32",
                  "grok_moe_forward_static"):
            getattr(h, n).restype = ctypes.c_int
        h.grok_moe_status_string.argtypes = [ctypes.c_int]
        h.grok_moe_status_string.restype = ctypes.c_char_p
        _lib_handle = h
    return _lib_handle


def grok_moe_status_string(code: int) -> str:
    return lib().grok_moe_status_string(int(code)).decode()


def grok_moe_workspace_bytes(T: int, d: int, f: int, E: int, k: int, act_dtype: int = BF16,
                             w_dtype: int = BF16) -> int:
    return int(lib().grok_moe_workspace_bytes(T, d, f, E, k, act_dtype, w_dtype))


def grok_moe_workspace_bytes_ex(x, router_w, w_gate, w_up, w_down, k: int = 2, **variant) -> int:
    """Workspace bytes of one grok_moe_forward_ex call with these tensors and variant knobs (sizing only:
    the 8-bit scales may be left out, and x stands in for out)."""
    a = make_args(x, router_w, w_gate, w_up, w_down, x, k, sizing=True, **variant)
    return int(lib().grok_moe_workspace_bytes_ex(ctypes.byref(a)))


def grok_moe_tile_rows(x, router_w, w_gate, w_up, w_down, k: int = 2, **variant) -> int:
    """Rows per grouped-GEMM tile that grok_moe_forward_ex runs for these tensors' sizes and dtypes and
    variant knobs (0 for fp32 activations or a rejected shape)."""
    a = make_args(x, router_w, w_gate, w_up, w_down, x, k, sizing=True, **variant)
    return int(lib().grok_moe_tile_rows(ctypes.byref(a)))


# ---------------------------------------------------------------- torch marshalling
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.int8:
        return I8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_tensors(named: Dict[str, object]):
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _shape(x, w_gate, router_w, n_shared: int = 0):
    """(T, d, f, E routed); the weights hold E + n_shared experts."""
    if x.dim() != 2 or w_gate.dim() != 3:
        raise ValueError("x must be [T, d] and w_gate [E, f, d]")
    T, d = x.shape
    Et, f, d2 = w_gate.shape
    E = Et - n_shared
    if d2 != d:
        raise ValueError(f"w_gate is [E, f, d] with d={d2}, x has d={d}")
    if E < 1:
        raise ValueError(f"w_gate holds {Et} experts, fewer than n_shared + 1 = {n_shared + 1}")
    if router_w is not None and tuple(router_w.shape) != (E, d):
        raise ValueError(f"router_w must be [E, d] = [{E}, {d}], got {tuple(router_w.shape)}")
    return T, d, f, E


def _validate(x, router_w, w_gate, w_up, w_down, out, k: int, scales=None, route_idx=None, route_gate=None,
              norm_pre=None, norm_post=None, n_shared: int = 0, router_bias=None, want_w=None,
              sizing: bool = False):
    """Checks every tensor's device, contiguity, shape and dtype against the layout of include/grok_moe.h
    before anything reaches the library (which sees only pointers and sizes). want_w: the weight dtype a
    plain entry point requires (None: any supported combination). sizing: the call only sizes a workspace
    (8-bit scales may be absent). Returns (T, d, f, E routed)."""
    torch = _torch()
    T, d, f, E = _shape(x, w_gate, router_w, n_shared)
    Et = E + n_shared
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    wdt = w_gate.dtype
    if want_w is not None and wdt != want_w:
        raise TypeError(f"this entry point takes {want_w} expert weights, got {wdt}")
    ok = {torch.bfloat16: (torch.bfloat16, torch.int8), torch.float32: (torch.float32,)}[x.dtype]
    if wdt not in ok:
        raise TypeError(f"{x.dtype} activations take expert weights of {ok}, got {wdt}")
    if tuple(w_up.shape) != (Et, f, d) or tuple(w_down.shape) != (Et, d, f):
        raise ValueError(f"w_up must be [E + n_shared, f, d] = [{Et}, {f}, {d}] and w_down [{Et}, {d}, {f}], got "
                         f"{tuple(w_up.shape)} and {tuple(w_down.shape)}")
    if w_up.dtype != wdt or w_down.dtype != wdt:
        raise TypeError(f"w_gate, w_up and w_down must share one dtype ({wdt}, {w_up.dtype}, {w_down.dtype})")
    if router_w is not None and router_w.dtype != x.dtype:
        raise TypeError(f"router_w must have the activation dtype {x.dtype}, got {router_w.dtype}")
    if tuple(out.shape) != (T, d) or out.dtype != x.dtype:
        raise ValueError(f"out must be [T, d] = [{T}, {d}] of dtype {x.dtype}, got {tuple(out.shape)} {out.dtype}")
    if wdt == torch.int8:
        n = 2 * Et * f + Et * d
        if scales is None and sizing:
            pass
        elif scales is None or scales.dtype != torch.float32 or scales.numel() != n:
            raise ValueError(f"int8 weights need float32 scales of 2*E*f + E*d = {n} values (gate | up | down)")
    elif scales is not None:
        raise ValueError("scales are only taken with int8 weights")
    if (route_idx is None) != (route_gate is None):
        raise ValueError("route_idx and route_gate go together")
    if route_idx is not None:
        if tuple(route_idx.shape) != (T, k) or route_idx.dtype != torch.int32:
            raise ValueError(f"route_idx must be [T, k] = [{T}, {k}] int32")
        if tuple(route_gate.shape) != (T, k) or route_gate.dtype != torch.float32:
            raise ValueError(f"route_gate must be [T, k] = [{T}, {k}] float32")
    elif router_w is None:
        raise ValueError("router_w is needed unless a routing (route_idx, route_gate) is given")
    if router_bias is not None and (tuple(router_bias.shape) != (E,) or router_bias.dtype != torch.float32):
        raise ValueError(f"router_bias must be [E] = [{E}] float32")
    if (norm_pre is None) != (norm_post is None):
        raise ValueError("norm_pre and norm_post go together")
    for name, g in (("norm_pre", norm_pre), ("norm_post", norm_post)):
        if g is not None and (tuple(g.shape) != (d,) or g.dtype != x.dtype):
            raise ValueError(f"{name} must be [d] = [{d}] of the activation dtype")
    _check_tensors(dict(x=x, router_w=router_w, w_gate=w_gate, w_up=w_up, w_down=w_down, out=out, scales=scales,
                        route_idx=route_idx, route_gate=route_gate, norm_pre=norm_pre, norm_post=norm_post,
                        router_bias=router_bias))
    return T, d, f, E


def make_args(x, router_w, w_gate, w_up, w_down, out, k: int, scales=None, route_idx=None,
              route_gate=None, activation: int = ACT_GELU, renormalize: bool = False,
              capacity_factor: float = 0.0, norm_pre=None, norm_post=None, norm_eps: float = 1e-5,
              n_shared: int = 0, router_bias=None, sizing: bool = False) -> Args:
    T, d, f, E = _validate(x, router_w, w_gate, w_up, w_down, out, k, scales, route_idx, route_gate, norm_pre,
                           norm_post, n_shared, router_bias, sizing=sizing)
    a = Args()
    a.x, a.router_w, a.w_gate, a.w_up, a.w_down = _ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down)
    a.scales, a.out = _ptr(scales), _ptr(out)
    a.T, a.d, a.f, a.E, a.k = T, d, f, E, k
    a.act_dtype = _dtype_code(x)
    a.w_dtype = _dtype_code(w_gate)
    a.route_idx, a.route_gate = _ptr(route_idx), _ptr(route_gate)
    a.activation, a.renormalize, a.capacity_factor = int(activation), int(bool(renormalize)), float(capacity_factor)
    a.norm_pre, a.norm_post, a.norm_eps = _ptr(norm_pre), _ptr(norm_post), float(norm_eps)
    a.n_shared, a.router_bias = int(n_shared), _ptr(router_bias)
    return a


def _raise(rc: int, where: str):
    if rc != OK:
        raise GrokMoeError(rc, where)


def grok_moe_forward(x, router_w, w_gate, w_up, w_down, out=None, k: int = 2, stream=None):
    """bf16 layer; allocates its workspace stream-ordered. Returns `out`."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    T, d, f, E = _validate(x, router_w, w_gate, w_up, w_down, out, k, want_w=torch.bfloat16)
    if x.dtype != torch.bfloat16:
        raise TypeError("grok_moe_forward takes bfloat16 activations")
    rc = lib().grok_moe_forward(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out), T, d,
                                f, E, k, _stream(stream))
    _raise(rc, "grok_moe_forward")
    return out


def grok_moe_forward_w8(x, router_w, w_gate, w_up, w_down, scales, out=None, k: int = 2, stream=None):
    """bf16 activations, int8 weights, fp32 scales [gate E*f | up E*f | down E*d]. Returns `out`."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    T, d, f, E = _validate(x, router_w, w_gate, w_up, w_down, out, k, scales=scales, want_w=torch.int8)
    rc = lib().grok_moe_forward_w8(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(scales),
                                   _ptr(out), T, d, f, E, k, _stream(stream))
    _raise(rc, "grok_moe_forward_w8")
    return out


def grok_moe_forward_f32(x, router_w, w_gate, w_up, w_down, out=None, k: int = 2, stream=None):
    """fp32 layer. Returns `out`."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    T, d, f, E = _validate(x, router_w, w_gate, w_up, w_down, out, k, want_w=torch.float32)
    rc = lib().grok_moe_forward_f32(_ptr(x), _ptr(router_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out), T,
                                    d, f, E, k, _stream(stream))
    _raise(rc, "grok_moe_forward_f32")
    return out


def grok_moe_forward_ex(x, router_w, w_gate, w_up, w_down, k: int = 2, scales=None, out=None, workspace=None,
                        route_idx=None, route_gate=None, debug: bool = False,
                        events: Optional[Sequence[object]] = None, stream=None, activation: int = ACT_GELU,
                        renormalize: bool = False, capacity_factor: float = 0.0, norm_pre=None, norm_post=None,
                        norm_eps: float = 1e-5, n_shared: int = 0, router_bias=None):
    """Layer with caller workspace. Returns (out, dbg) where dbg holds the routing intermediates
    (idx, gate, counts, offsets, perm, pos, and u with the sandwich norms) as device tensors when
    debug=True, else {}.
    `events`: up to 6 raw hipEvent_t handles (see `HipEvents`) recorded before each stage and after the last.
    Variants: activation (ACT_GELU / ACT_SILU), renormalize, capacity_factor, norm_pre/norm_post/norm_eps
    (the sandwich sub-layer out = x + RMSNorm(MoE(RMSNorm(x)))), n_shared (shared experts stored after the
    routed ones in the weights; the debug routing then has k + n_shared slots) and router_bias."""
    torch = _torch()
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    a = make_args(x, router_w, w_gate, w_up, w_down, out, k, scales, route_idx, route_gate, activation,
                  renormalize, capacity_factor, norm_pre, norm_post, norm_eps, n_shared, router_bias)
    need = int(lib().grok_moe_workspace_bytes_ex(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    dbg, dptr = _debug(a, k, n_shared, norm_pre is not None, dev, debug, events)
    rc = lib().grok_moe_forward_ex(ctypes.byref(a), workspace.data_ptr(), workspace.numel(), dptr,
                                   _stream(stream))
    _raise(rc, "grok_moe_forward_ex")
    return out, dbg


def grok_moe_forward_static(x, router_w, w_gate, w_up, w_down, k: int = 2, scales=None, out=None,
                            route_idx=None, route_gate=None, debug: bool = False,
                            events: Optional[Sequence[object]] = None, stream=None, activation: int = ACT_GELU,
                            renormalize: bool = False, capacity_factor: float = 0.0, norm_pre=None,
                            norm_post=None, norm_eps: float = 1e-5, n_shared: int = 0, router_bias=None):
    """grok_moe_forward_ex without a workspace argument: the library uses its static per-device workspace
    (STATIC_WORKSPACE_BYTES; larger shapes raise GrokMoeError with EWORKSPACE). Calls that overlap in time on
    one device race on that workspace. Returns (out, dbg) like grok_moe_forward_ex (`out` must be given
    when the caller cannot allocate)."""
    torch = _torch()
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    a = make_args(x, router_w, w_gate, w_up, w_down, out, k, scales, route_idx, route_gate, activation,
                  renormalize, capacity_factor, norm_pre, norm_post, norm_eps, n_shared, router_bias)
    dbg, dptr = _debug(a, k, n_shared, norm_pre is not None, dev, debug, events)
    rc = lib().grok_moe_forward_static(ctypes.byref(a), dptr, _stream(stream))
    _raise(rc, "grok_moe_forward_static")
    return out, dbg


def _debug(a, k, n_shared, sandwich, dev, debug, events):
    """Debug struct (device arrays for the routing intermediates, event handles) or (dict(), None)."""
    torch = _torch()
    dbg = {}
    if not (debug or events):
        return dbg, None
    d = Debug()
    if debug:
        T, E, K = a.T, a.E + n_shared, k + n_shared
        dbg = dict(idx=torch.full((T, K), -7, dtype=torch.int32, device=dev),
                   gate=torch.full((T, K), -7.0, dtype=torch.float32, device=dev),
                   counts=torch.full((E,), -7, dtype=torch.int32, device=dev),
                   offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
                   perm=torch.full((T * K,), -7, dtype=torch.int32, device=dev),
                   pos=torch.full((T, K), -7, dtype=torch.int32, device=dev))
        if sandwich:
            dbg["u"] = torch.empty((a.T, a.d), dtype=torch.bfloat16 if a.act_dtype == BF16 else torch.float32,
                                   device=dev)
        for name, t in dbg.items():
            setattr(d, name, t.data_ptr())
    if events:
        for i, ev in enumerate(events[:6]):
            if ev:
                d.events[i] = ctypes.c_void_p(int(ev))
    return dbg, ctypes.byref(d)


# ---------------------------------------------------------------- HIP events (timing plumbing)
class HipEvents:
    """A set of hipEvent_t handles made with the HIP runtime, for per-stage timing on any stream."""

    def __init__(self, n: int):
        self._rt = ctypes.CDLL("libamdhip64.so")
        self._rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self._rt.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        """Milliseconds between event i and event j (synchronises on event j)."""
        self._rt.hipEventSynchronize(self.handles[j])
        ms = ctypes.c_float()
        rc = self._rt.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self._rt.hipEventDestroy(h)
        self.handles = []
