"""Seeded synthetic inputs for the Grok-1 MoE feed-forward layer.

This package makes input data only; it holds none of the layer's arithmetic.
The CPU oracle and the GPU library both take their inputs from here, so the
two sides always see identical bits.

Workload shapes follow the pages' Grok-1 configuration: hidden size
d = 48*128 = 6144, 8 experts with 2 selected per token, expert width
f = 8*6144*2/3 = 32768 (Grok-1 book ch. 1, section 1.2, the run.py config and
the parameter arithmetic under it), one full context of 8192 tokens, and an
8-bit weight variant (same section, the INT8 box; field guide, spec table).

Storage layouts (all row-major, contiguous):

* ``x``        [T][d]       activations (bf16, or f32 for the tiny workload)
* ``router_w`` [E][d]       row e holds the d router weights of expert e
* ``w_gate``   [E][f][d]    row j of expert e holds the d input weights of
  gate channel j (output-channel-major, like a torch Linear weight)
* ``w_up``     [E][f][d]    same for the linear branch
* ``w_down``   [E][d][f]    row i of expert e holds the f weights of output i
* ``scales``   fp32, packed [gate: E*f | up: E*f | down: E*d], one per output
  channel (8-bit workload only); the real weight is q * scale.

Tensor ids for the counter-based generator: x=0, router=1, gate=2, up=3,
down=4, pre-norm weights=5, post-norm weights=6 (7: the test-only random
scales), router selection bias=8.

Variants beside the Grok-1 layer: the Mixtral 8x22B shape (d = 6144,
f = 16384, 8 experts, top-2; book ch. 10, section 10.1 table) with SiLU
experts and renormalised gates; the sandwich sub-layer (RMSNorm weights
before and after the MoE); a capacity factor; the fine-grained DeepSeek-V3
layout (d = 7168, 256 routed experts of width 2048, top-8, one shared expert,
a per-expert selection bias; book ch. 10, section 10.1 table and sections
10.3.2 and 10.11.4), whose shared expert's weights follow the routed ones.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_gen.c")
_LIB = os.path.join(_HERE, "libsynthetic.so")
_lib_handle = None

TID_X, TID_ROUTER, TID_GATE, TID_UP, TID_DOWN, TID_NORM_PRE, TID_NORM_POST = 0, 1, 2, 3, 4, 5, 6
TID_ROUTER_BIAS = 8
ROUTER_BIAS_STD = 1e-3   # selection bias scale, against probabilities of about 1/256


def build(force: bool = True) -> str:
    """Compile the generator with the host C compiler (no GPU code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, u64, u32, dbl, cint = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_int
        vp = ctypes.c_void_p
        lib.syn_normal_f32.argtypes = [vp, i64, u64, u32, dbl, cint]
        lib.syn_normal_bf16.argtypes = [vp, i64, u64, u32, dbl, cint]
        lib.syn_uniform_i8.argtypes = [vp, i64, u64, u32, cint]
        lib.syn_philox4x32_10.argtypes = [vp, vp, vp]
        for fn in (lib.syn_normal_f32, lib.syn_normal_bf16, lib.syn_uniform_i8, lib.syn_philox4x32_10):
            fn.restype = None
        _lib_handle = lib
    return _lib_handle


def host_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _lib().syn_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal(shape, seed: int, tensor_id: int, scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Normals N(0, scale^2). bf16 tensors are returned as uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        _lib().syn_normal_bf16(out.ctypes.data, n, seed, tensor_id, float(scale), host_threads())
    elif dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        _lib().syn_normal_f32(out.ctypes.data, n, seed, tensor_id, float(scale), host_threads())
    else:
        raise ValueError(f"unknown dtype {dtype}")
    return out


def uniform_i8(shape, seed: int, tensor_id: int) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.int8)
    _lib().syn_uniform_i8(out.ctypes.data, n, seed, tensor_id, host_threads())
    return out


# ---------------------------------------------------------------- bf16 helpers
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even), as uint16 bit patterns."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- workloads
@dataclass
class Workload:
    """One synthetic MoE-layer input set. Arrays are host numpy arrays."""
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    act_dtype: str          # "bf16" | "f32"
    w_dtype: str            # "bf16" | "f32" | "i8"
    x: np.ndarray
    router_w: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    scales: Optional[np.ndarray] = None
    seed: int = 0
    notes: Dict[str, str] = field(default_factory=dict)
    activation: str = "gelu"            # "gelu" | "silu"
    renormalize: bool = False
    capacity_factor: float = 0.0        # 0: no cap
    norm_pre: Optional[np.ndarray] = None   # [d], activation dtype (sandwich sub-layer)
    norm_post: Optional[np.ndarray] = None
    norm_eps: float = 1e-5
    n_shared: int = 0                   # shared experts stored after the E routed ones
    router_bias: Optional[np.ndarray] = None  # [E] fp32 selection bias

    @property
    def weight_bytes(self) -> int:
        return int(self.w_gate.nbytes + self.w_up.nbytes + self.w_down.nbytes)


# name -> (T, d, f, E, k, act dtype, weight dtype, skew)
WORKLOADS = {
    # Tiny fp32 layer: T=64, d=256, f=1024, E=8, top-2.
    "tiny_f32": (64, 256, 1024, 8, 2, "f32", "f32", False),
    # Grok-1-shape decode step: 8 tokens.
    "decode": (8, 6144, 32768, 8, 2, "bf16", "bf16", False),
    # Grok-1-shape prefill of one full 8192-token context.
    "prefill": (8192, 6144, 32768, 8, 2, "bf16", "bf16", False),
    # Grok-1-shape layer with 8-bit expert weights, 256 tokens.
    "int8": (256, 6144, 32768, 8, 2, "bf16", "i8", False),
    # Grok-1-shape layer with router logits biased toward experts 0 and 1.
    "skew": (2048, 6144, 32768, 8, 2, "bf16", "bf16", True),
    # Mixtral 8x22B-shape decode step and full-context prefill (SiLU, renormalised gates).
    "mixtral_decode": (8, 6144, 16384, 8, 2, "bf16", "bf16", False),
    "mixtral_prefill": (8192, 6144, 16384, 8, 2, "bf16", "bf16", False),
    # DeepSeek-V3-shape fine-grained layer: 256 routed experts of width 2048, top-8, plus one shared expert.
    "dsv3_decode": (8, 7168, 2048, 256, 8, "bf16", "bf16", False),
    "dsv3_prefill": (8192, 7168, 2048, 256, 8, "bf16", "bf16", False),
}

# name -> variant knobs that differ from the Grok-1 layer
VARIANTS = {
    "mixtral_decode": dict(activation="silu", renormalize=True),
    "mixtral_prefill": dict(activation="silu", renormalize=True),
    "dsv3_decode": dict(activation="silu", renormalize=True, n_shared=1, router_bias=True),
    "dsv3_prefill": dict(activation="silu", renormalize=True, n_shared=1, router_bias=True),
}


def norm_weights(d: int, seed: int, dtype: str = "bf16"):
    """RMSNorm weights of the sandwich sub-layer: 1 + 0.1 z per channel, z ~ N(0, 1), rounded to `dtype`."""
    out = []
    for tid in (TID_NORM_PRE, TID_NORM_POST):
        g = 1.0 + normal((d,), seed, tid, 0.1, "f32")
        out.append(g.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(g.astype(np.float32)))
    return out[0], out[1]

# Skew construction: feature d-1 of every token is 1.0 and the router row of
# expert e carries SKEW_BIAS[e] at feature d-1, so logit e gains exactly that
# bias (1.0, 3.0 and 1.5 are exact in bf16).
SKEW_BIAS = (3.0, 1.5)


def make(name: str = "decode", seed: int = 0, T: Optional[int] = None, d: Optional[int] = None,
         f: Optional[int] = None, E: Optional[int] = None, k: Optional[int] = None,
         act_dtype: Optional[str] = None, w_dtype: Optional[str] = None,
         skew: Optional[bool] = None, with_weights: bool = True, activation: Optional[str] = None,
         renormalize: Optional[bool] = None, capacity_factor: Optional[float] = None,
         sandwich: bool = False, norm_eps: float = 1e-5, n_shared: Optional[int] = None,
         router_bias: Optional[bool] = None) -> Workload:
    """Build a named workload; any size, dtype or variant knob can be overridden (for small parity cases).

    with_weights=False leaves the expert weights as empty placeholders (routing-only checks).
    sandwich=True adds the RMSNorm weights of the sandwich sub-layer; n_shared appends that many shared
    experts to the weights; router_bias=True draws a per-expert selection bias.
    """
    T0, d0, f0, E0, k0, a0, w0, s0 = WORKLOADS[name]
    T = T0 if T is None else T
    d = d0 if d is None else d
    f = f0 if f is None else f
    E = E0 if E is None else E
    k = k0 if k is None else k
    act = a0 if act_dtype is None else act_dtype
    wdt = w0 if w_dtype is None else w_dtype
    skew = s0 if skew is None else skew
    var = dict(activation="gelu", renormalize=False, capacity_factor=0.0, n_shared=0, router_bias=False)
    var.update(VARIANTS.get(name, {}))
    for key, val in (("activation", activation), ("renormalize", renormalize), ("capacity_factor", capacity_factor),
                     ("n_shared", n_shared), ("router_bias", router_bias)):
        if val is not None:
            var[key] = val
    Et = E + var["n_shared"]   # experts in the weight tensors

    x = normal((T, d), seed, TID_X, 1.0, act)
    rdt = "f32" if act == "f32" else "bf16"
    router_w = normal((E, d), seed, TID_ROUTER, 1.0 / math.sqrt(d), rdt)
    scales = None
    if not with_weights:
        w_gate = w_up = w_down = np.zeros((0,), np.uint16)
    elif wdt == "i8":
        w_gate = uniform_i8((Et, f, d), seed, TID_GATE)
        w_up = uniform_i8((Et, f, d), seed, TID_UP)
        w_down = uniform_i8((Et, d, f), seed, TID_DOWN)
        s_in = np.float32(1.0 / (127.0 * math.sqrt(d)))
        s_ff = np.float32(1.0 / (127.0 * math.sqrt(f)))
        scales = np.concatenate([np.full(Et * f, s_in, np.float32), np.full(Et * f, s_in, np.float32),
                                 np.full(Et * d, s_ff, np.float32)])
    else:
        w_gate = normal((Et, f, d), seed, TID_GATE, 1.0 / math.sqrt(d), wdt)
        w_up = normal((Et, f, d), seed, TID_UP, 1.0 / math.sqrt(d), wdt)
        w_down = normal((Et, d, f), seed, TID_DOWN, 1.0 / math.sqrt(f), wdt)
    notes = {}
    if skew:
        one = np.float32(1.0)
        if act == "f32":
            x[:, d - 1] = one
        else:
            x[:, d - 1] = f32_to_bf16_bits(np.array([one]))[0]
        bias = np.zeros(E, np.float32)
        for e, b in enumerate(SKEW_BIAS[:E]):
            bias[e] = b
        if rdt == "f32":
            router_w[:, d - 1] = bias
        else:
            router_w[:, d - 1] = f32_to_bf16_bits(bias)
        notes["skew"] = "x[:, d-1] = 1.0; router_w[:, d-1] = (+3.0, +1.5, 0, ...)"
    if var["activation"] not in ("gelu", "silu"):
        raise ValueError(f"unknown activation {var['activation']}")
    norm_pre = norm_post = None
    if sandwich:
        norm_pre, norm_post = norm_weights(d, seed, act)
    var["router_bias"] = (normal((E,), seed, TID_ROUTER_BIAS, ROUTER_BIAS_STD, "f32")
                          if var["router_bias"] else None)
    return Workload(name=name, T=T, d=d, f=f, E=E, k=k, act_dtype=act, w_dtype=wdt, x=x,
                    router_w=router_w, w_gate=w_gate, w_up=w_up, w_down=w_down, scales=scales,
                    seed=seed, notes=notes, norm_pre=norm_pre, norm_post=norm_post, norm_eps=norm_eps, **var)


def random_scales(E: int, d: int, f: int, seed: int, tensor_id: int = 7) -> np.ndarray:
    """Per-output-channel scales base * 2^u, u ~ U[-1, 1] (distinct per channel), packed like `scales`.

    Used by tests to pin scale indexing: the workload's own scales are equal per matrix.
    """
    n = 2 * E * f + E * d
    z = normal((n,), seed, tensor_id, 1.0, "f32").astype(np.float64)
    u = np.tanh(z)  # in (-1, 1)
    base = np.concatenate([np.full(2 * E * f, 1.0 / (127.0 * math.sqrt(d))),
                           np.full(E * d, 1.0 / (127.0 * math.sqrt(f)))])
    return (base * np.exp2(u)).astype(np.float32)
