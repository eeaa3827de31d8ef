"""Host-side checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before anything touches a GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import mixture_experts_transformer_gemm_amd as gm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grok_moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(grok_moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_names():
    decl = declared_functions()
    assert decl == sorted(gm.EXPORTED), decl


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gm.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_is_gfx950_code():
    blob = open(gm.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        s = gm.grok_moe_status_string(code)
        assert s and s != "unknown status"
    assert gm.grok_moe_status_string(7) == "unknown status"


def test_workspace_bytes():
    # decode shape: idx/gate/perm/pos + H [16, f] bf16 + split-K Y partials
    ws = gm.grok_moe_workspace_bytes(8, 6144, 32768, 8, 2)
    assert ws >= 16 * 32768 * 2 + 16 * 6144 * 4
    # prefill: H [16384, 32768] bf16 dominates; Y [2][16384, 6144] fp32 (8 experts x 7 row tiles of 320 x 24
    # channel tiles = 1,344 down tiles leave the last of 256 workgroup rounds 25% full, so the reduction runs
    # in two splits); u [8192, 6144] bf16 for the sandwich norms
    ws = gm.grok_moe_workspace_bytes(8192, 6144, 32768, 8, 2)
    assert 16384 * 32768 * 2 + 2 * 16384 * 6144 * 4 <= ws
    assert ws < 16384 * 32768 * 2 + 2 * 16384 * 6144 * 4 + 8192 * 6144 * 2 + (1 << 20)
    # 16,384 tokens: 8 x 13 row tiles x 24 = 2,496 down tiles (9.75 rounds: the last 75% full), one split
    ws = gm.grok_moe_workspace_bytes(16384, 6144, 32768, 8, 2)
    assert 32768 * 32768 * 2 + 32768 * 6144 * 4 <= ws < 32768 * 32768 * 2 + 2 * 32768 * 6144 * 4
    # 32,768 tokens: 8 x 26 x 24 = 4,992 down tiles (19.5 rounds), two splits
    ws = gm.grok_moe_workspace_bytes(32768, 6144, 32768, 8, 2)
    assert ws >= 65536 * 32768 * 2 + 2 * 65536 * 6144 * 4
    assert gm.grok_moe_workspace_bytes(0, 6144, 32768, 8, 2) > 0
    # invalid / unsupported shapes report 0
    assert gm.grok_moe_workspace_bytes(8, 6144, 32768, 8, 9) == 0          # k > E
    assert gm.grok_moe_workspace_bytes(8, 6100, 32768, 8, 2) == 0          # d % 64
    # widths that are multiples of 64 (d) and 128 (f) only: every path takes them, with bf16 and 8-bit
    # weights (a Mixtral-8x7B-like 4096 x 14336, and 6208 x 1408)
    for T in (8, 200, 2100):
        for wdt in (gm.BF16, gm.I8):
            for d, f in ((320, 384), (6208, 1408), (4096, 14336)):
                assert gm.grok_moe_workspace_bytes(T, d, f, 8, 2, gm.BF16, wdt) >= 2 * T * f * 2, (T, d, f, wdt)
    assert gm.grok_moe_workspace_bytes(8, 6144, 32768, 257, 2) == 0        # E > 256
    assert gm.grok_moe_workspace_bytes(8, 64, 64, 65, 2, gm.F32, gm.F32) == 0   # fp32 router: E <= 64
    # many experts: the router's split-K logits [S][T][E] fp64 are part of the workspace
    assert gm.grok_moe_workspace_bytes(8192, 7168, 2048, 256, 8) >= 8192 * 256 * 8
    # fine-grained decode (256 experts of width 2048, top-8, 8 tokens: about 58 experts hit, 1,869
    # gate/up workgroups): the gate/up reduction runs in two splits whose fp32 sums [2][64][4096]
    # are part of the workspace, next to Y [64][7168] fp32
    assert gm.grok_moe_workspace_bytes(8, 7168, 2048, 256, 8) >= 2 * 64 * 4096 * 4 + 64 * 7168 * 4
    # 16 tokens (about 103 experts hit, 3,295 workgroups): one split, no such buffer (with it the
    # workspace would hold at least G [2][128][4096] and Y [128][7168] fp32)
    assert gm.grok_moe_workspace_bytes(16, 7168, 2048, 256, 8) < 2 * 128 * 4096 * 4 + 128 * 7168 * 4
    assert gm.grok_moe_workspace_bytes(8, 6144, 32768, 8, 2, gm.F32, gm.BF16) == 0   # dtype combo


def _args(**kw):
    a = gm.Args()
    base = dict(x=0x10000, router_w=0x20000, w_gate=0x30000, w_up=0x40000, w_down=0x50000, scales=None,
                out=0x60000, T=8, d=256, f=512, E=8, k=2, act_dtype=gm.BF16, w_dtype=gm.BF16, route_idx=None,
                route_gate=None, activation=gm.ACT_GELU, renormalize=0, capacity_factor=0.0, norm_pre=None,
                norm_post=None, norm_eps=1e-5, n_shared=0, router_bias=None)
    base.update(kw)
    for n, v in base.items():
        setattr(a, n, v)
    return a


def _call(a, ws=0x1000000, ws_bytes=1 << 40):
    # every case below is rejected before the first HIP call
    return gm.lib().grok_moe_forward_ex(ctypes.byref(a), ws, ws_bytes, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), gm.EINVAL),
    (dict(out=None), gm.EINVAL),
    (dict(w_down=None), gm.EINVAL),
    (dict(router_w=None), gm.EINVAL),
    (dict(route_idx=0x70000), gm.EINVAL),            # routing override without gates
    (dict(T=-1), gm.EINVAL),
    (dict(k=0), gm.EINVAL),
    (dict(k=9, E=8), gm.EINVAL),
    (dict(E=0), gm.EINVAL),
    (dict(act_dtype=gm.F32), gm.EINVAL),             # f32 activations with bf16 weights
    (dict(act_dtype=5), gm.EINVAL),
    (dict(w_dtype=gm.I8), gm.EINVAL),                # int8 without scales
    (dict(E=257, k=2), gm.EUNSUPPORTED),
    (dict(E=65, k=2, act_dtype=gm.F32, w_dtype=gm.F32), gm.EUNSUPPORTED),
    (dict(E=16, k=9), gm.EUNSUPPORTED),
    (dict(n_shared=5), gm.EUNSUPPORTED),
    (dict(n_shared=-1), gm.EINVAL),
    (dict(router_bias=0x80004), gm.EALIGN),
    (dict(d=200), gm.EUNSUPPORTED),
    (dict(d=352), gm.EUNSUPPORTED),                  # bf16 / 8-bit weights: d % 64
    (dict(f=320), gm.EUNSUPPORTED),                  # f % 128
    (dict(T=(1 << 20) + 1), gm.EUNSUPPORTED),
    (dict(x=0x10008), gm.EALIGN),
    (dict(w_up=0x40004), gm.EALIGN),
    (dict(out=0x60002), gm.EALIGN),
    # variants
    (dict(activation=2), gm.EINVAL),
    (dict(activation=-1), gm.EINVAL),
    (dict(capacity_factor=-0.5), gm.EINVAL),
    (dict(capacity_factor=float("nan")), gm.EINVAL),
    (dict(capacity_factor=float("inf")), gm.EINVAL),
    (dict(norm_pre=0x80000), gm.EINVAL),              # one norm without the other
    (dict(norm_post=0x90000), gm.EINVAL),
    (dict(norm_pre=0x80000, norm_post=0x90000, norm_eps=-1e-5), gm.EINVAL),
    (dict(norm_pre=0x80000, norm_post=0x90000, norm_eps=float("nan")), gm.EINVAL),
    (dict(norm_pre=0x80008, norm_post=0x90000), gm.EALIGN),
])
def test_validation_errors(kw, code):
    assert _call(_args(**kw)) == code


def test_variant_arguments_reach_the_workspace_check():
    # valid variant knobs pass validation (the call then stops at the missing workspace)
    for kw in (dict(activation=gm.ACT_SILU, renormalize=1), dict(capacity_factor=1.25),
               dict(norm_pre=0x80000, norm_post=0x90000, norm_eps=0.0), dict(n_shared=4),
               dict(E=256, k=8, n_shared=1, router_bias=0x80000)):
        assert _call(_args(**kw), ws=0, ws_bytes=0) == gm.EWORKSPACE


def test_workspace_bytes_ex_counts_shared_experts():
    a = _args(T=64, d=7168, f=2048, E=256, k=8)
    base = gm.lib().grok_moe_workspace_bytes_ex(ctypes.byref(a))
    assert base == gm.grok_moe_workspace_bytes(64, 7168, 2048, 256, 8)
    a.n_shared = 1
    more = gm.lib().grok_moe_workspace_bytes_ex(ctypes.byref(a))
    assert more >= base + 64 * 2048 * 2          # one more H row per token at least
    assert _call(a, ws=0x1000000, ws_bytes=base) == gm.EWORKSPACE
    a.k = 9
    assert gm.lib().grok_moe_workspace_bytes_ex(ctypes.byref(a)) == 0


@pytest.mark.parametrize("kw,rows", [
    (dict(T=8, d=6144, f=32768), 16),                                   # Grok-1 decode: streaming, 16-row chunks
    (dict(T=64, d=6144, f=32768), 64),
    (dict(T=256, d=6144, f=32768, w_dtype=gm.I8), 128),                # 8-bit streaming, 128-row chunks
    (dict(T=8192, d=6144, f=32768), 320),                               # prefill: ping-pong 320-row tiles
    (dict(T=8192, d=6144, f=32768, w_dtype=gm.I8), 256),                # 8-bit: tiled 256-row tiles
    (dict(T=1100, d=256, f=512), 320),                                  # 275 rows per expert
    (dict(T=800, d=256, f=512), 320),                                   # 200 rows per expert: ping-pong
    (dict(T=700, d=256, f=512), 256),                                   # 175 rows per expert: tiled
    (dict(T=772, d=256, f=512), 320),                                   # 193 rows per expert: ping-pong
    (dict(T=768, d=256, f=512), 256),                                   # 192 rows per expert: tiled
    (dict(T=8192, d=7168, f=2048, E=256, k=8, n_shared=1), 320),        # 287 rows per expert
    (dict(T=300, d=256, f=512, w_dtype=gm.I8), 128),
    (dict(T=64, d=256, f=512, act_dtype=gm.F32, w_dtype=gm.F32), 0),   # fp32: no row tiles
    (dict(T=8, k=9), 0),                                                # rejected shape
])
def test_tile_rows(kw, rows):
    assert gm.lib().grok_moe_tile_rows(ctypes.byref(_args(**kw))) == rows


def test_ctypes_structs_match_the_header(tmp_path):
    # offsets and sizes of grok_moe_args / grok_moe_debug as the C compiler lays them out
    fields = {"grok_moe_args": gm.Args, "grok_moe_debug": gm.Debug}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "grok_moe.h"', "int main(void) {"]
    for cname, py in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    got = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        cname, fname, val = line.split()
        got[(cname, fname)] = int(val)
    for cname, py in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_workspace_errors():
    a = _args()
    need = gm.grok_moe_workspace_bytes(8, 256, 512, 8, 2)
    assert _call(a, ws=0x1000000, ws_bytes=need - 1) == gm.EWORKSPACE
    assert _call(a, ws=0, ws_bytes=need) == gm.EWORKSPACE
    assert _call(a, ws=0x1000010, ws_bytes=need) == gm.EALIGN


def test_zero_tokens_is_a_noop():
    # T = 0: valid shape, nothing enqueued, OK returned even with null tensors
    assert _call(_args(T=0, x=None, out=None), ws=0, ws_bytes=0) == gm.OK


def test_f32_shapes():
    a = _args(act_dtype=gm.F32, w_dtype=gm.F32, d=24, f=20)
    assert _call(a, ws=0x1000000, ws_bytes=16) == gm.EWORKSPACE   # valid shape, reaches the workspace check
    assert _call(_args(act_dtype=gm.F32, w_dtype=gm.F32, d=12)) == gm.EUNSUPPORTED


def test_plain_entry_points_validate_first():
    lib = gm.lib()
    assert lib.grok_moe_forward(None, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 8, 256, 512, 8, 2, None) \
        == gm.EINVAL
    assert lib.grok_moe_forward_w8(0x10000, 0x20000, 0x30000, 0x40000, 0x50000, None, 0x60000, 8, 256, 512, 8, 2,
                                   None) == gm.EINVAL
    assert lib.grok_moe_forward_f32(0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 8, 10, 512, 8, 2,
                                    None) == gm.EUNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(gm, "_lib_handle", None)
    monkeypatch.setattr(gm, "LIB_PATH", "/nonexistent/libgrok_moe.so")
    with pytest.raises(RuntimeError, match="missing"):
        gm.lib()


def test_build_rejects_scratch_kernels():
    # the build fails when the compiler's resource-usage remark reports scratch memory for a kernel
    from mixture_experts_transformer_gemm_amd.build import scratch_kernels
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: _Z1av [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:2:1: remark: Function Name: _Z1bv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:2:1: remark:     ScratchSize [bytes/lane]: 336 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_kernels(remarks) == [("_Z1bv", 336)]


def test_static_workspace_holds_the_grok1_layer_up_to_128_tokens():
    # the header's statement about GROK_MOE_STATIC_WORKSPACE_BYTES (64 MiB)
    assert gm.STATIC_WORKSPACE_BYTES == 64 << 20
    for wdt in (gm.BF16, gm.I8):
        for T in (1, 8, 64, 65, 128):
            assert 0 < gm.grok_moe_workspace_bytes(T, 6144, 32768, 8, 2, gm.BF16, wdt) <= gm.STATIC_WORKSPACE_BYTES


def test_static_entry_point_validates_before_touching_a_gpu():
    a = _args(T=8, d=256, f=256, E=8, k=9)
    assert gm.lib().grok_moe_forward_static(ctypes.byref(a), None, None) == gm.EINVAL
    a = _args(T=0, d=256, f=256, E=8, k=2)
    assert gm.lib().grok_moe_forward_static(ctypes.byref(a), None, None) == gm.OK


def _cpu_layer(T=4, d=64, f=128, E=4, wdt="bf16"):
    torch = pytest.importorskip("torch")
    adt = torch.float32 if wdt == "f32" else torch.bfloat16
    w = {"bf16": torch.bfloat16, "f32": torch.float32, "i8": torch.int8}[wdt]
    t = dict(x=torch.zeros(T, d, dtype=adt), router_w=torch.zeros(E, d, dtype=adt),
             w_gate=torch.zeros(E, f, d, dtype=w), w_up=torch.zeros(E, f, d, dtype=w),
             w_down=torch.zeros(E, d, f, dtype=w), out=torch.zeros(T, d, dtype=adt))
    return torch, t


@pytest.mark.parametrize("case", ["out_shape", "out_dtype", "up_shape", "down_shape", "down_dtype", "router_dtype",
                                  "scales_len", "scales_dtype", "scales_missing", "scales_bf16", "route_idx_dtype",
                                  "route_gate_shape", "route_alone", "norm_alone", "act_dtype"])
def test_binding_rejects_bad_tensors_before_the_library(case):
    # every tensor's shape and dtype is checked before a pointer reaches the library, which cannot check
    # sizes; these raise on host tensors, before the device check, so no GPU is needed
    wdt = "i8" if case.startswith("scales") and case != "scales_bf16" else "bf16"
    torch, t = _cpu_layer(wdt=wdt)
    T, d, f, E = 4, 64, 128, 4
    kw = {}
    if wdt == "i8":
        kw["scales"] = torch.zeros(2 * E * f + E * d, dtype=torch.float32)
    if case == "out_shape":
        t["out"] = torch.zeros(T, d + 1, dtype=torch.bfloat16)
    elif case == "out_dtype":
        t["out"] = torch.zeros(T, d, dtype=torch.float32)
    elif case == "up_shape":
        t["w_up"] = torch.zeros(E, f, d + 8, dtype=torch.bfloat16)
    elif case == "down_shape":
        t["w_down"] = torch.zeros(E, f, d, dtype=torch.bfloat16)
    elif case == "down_dtype":
        t["w_down"] = torch.zeros(E, d, f, dtype=torch.float32)
    elif case == "router_dtype":
        t["router_w"] = torch.zeros(E, d, dtype=torch.float32)
    elif case == "scales_len":
        kw["scales"] = torch.zeros(2 * E * f + E * d - 1, dtype=torch.float32)
    elif case == "scales_dtype":
        kw["scales"] = torch.zeros(2 * E * f + E * d, dtype=torch.bfloat16)
    elif case == "scales_missing":
        kw.pop("scales")
    elif case == "scales_bf16":
        kw["scales"] = torch.zeros(2 * E * f + E * d, dtype=torch.float32)
    elif case == "route_idx_dtype":
        kw["route_idx"] = torch.zeros(T, 2, dtype=torch.int64)
        kw["route_gate"] = torch.zeros(T, 2, dtype=torch.float32)
    elif case == "route_gate_shape":
        kw["route_idx"] = torch.zeros(T, 2, dtype=torch.int32)
        kw["route_gate"] = torch.zeros(T, 3, dtype=torch.float32)
    elif case == "route_alone":
        kw["route_idx"] = torch.zeros(T, 2, dtype=torch.int32)
    elif case == "norm_alone":
        kw["norm_pre"] = torch.zeros(d, dtype=torch.bfloat16)
    elif case == "act_dtype":
        t["x"] = torch.zeros(T, d, dtype=torch.float16)
    with pytest.raises((ValueError, TypeError)) as ei:
        gm.make_args(t["x"], t["router_w"], t["w_gate"], t["w_up"], t["w_down"], t["out"], 2, **kw)
    assert "device" not in str(ei.value)


def test_plain_wrappers_check_the_weight_dtype():
    torch, t = _cpu_layer(wdt="f32")
    with pytest.raises(TypeError):
        gm.grok_moe_forward(t["x"], t["router_w"], t["w_gate"], t["w_up"], t["w_down"], out=t["out"])
    with pytest.raises(TypeError):
        gm.grok_moe_forward_w8(t["x"], t["router_w"], t["w_gate"], t["w_up"], t["w_down"], None, out=t["out"])
    torch, t = _cpu_layer(wdt="bf16")
    with pytest.raises(TypeError):
        gm.grok_moe_forward_f32(t["x"], t["router_w"], t["w_gate"], t["w_up"], t["w_down"], out=t["out"])
    t["out"] = torch.zeros(3, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gm.grok_moe_forward(t["x"], t["router_w"], t["w_gate"], t["w_up"], t["w_down"], out=t["out"])
