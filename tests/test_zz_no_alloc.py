"""The allocation-free entry point, grok_moe_forward_static, through the C ABI: its
output and routing intermediates equal grok_moe_forward_ex's on the same inputs (the
same kernels and plan, so bit for bit), on two calls in a row with the second one
smaller (the static workspace keeps the first call's contents), on the
weight-streaming and the tiled paths, and within the oracle's tolerance; a shape
needing more than the static workspace is refused before anything is enqueued."""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import TOL, dev_workload, normwise_err

torch = pytest.importorskip("torch")
import mixture_experts_transformer_gemm_amd as gm  # noqa: E402

pytestmark = pytest.mark.gpu


def _both(w):
    dev = dev_workload(w, torch)
    args = (dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"])
    ref, dref = gm.grok_moe_forward_ex(*args, k=w.k, scales=dev["scales"], debug=True)
    out = torch.full_like(dev["x"], float("nan"))
    got, dgot = gm.grok_moe_forward_static(*args, k=w.k, scales=dev["scales"], out=out, debug=True)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    for name in ("idx", "gate", "counts", "offsets", "perm", "pos"):
        assert torch.equal(dgot[name], dref[name]), name
    a = got.view(torch.int16).cpu().numpy()
    b = ref.view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    probs, _, _ = oracle.route(w.x, w.router_w, w.k)
    gidx = dgot["idx"].cpu().numpy()
    gates = np.take_along_axis(probs, gidx.astype(np.int64), 1)
    refo = oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, gidx, gates, scales=w.scales)
    err = normwise_err(got.float().cpu().numpy().astype(np.float64), refo)
    tol = TOL["i8" if w.w_dtype == "i8" else "bf16"]
    print(f"[no-alloc] T={w.T} d={w.d} f={w.f} {w.w_dtype}: bit-identical to the workspace form, normwise "
          f"error {err:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("first,second", [((300, 512, 768), (40, 256, 512)), ((64, 256, 512), (7, 256, 256))])
def test_static_matches_workspace_form_twice(first, second):
    # the first call fills the static workspace; the second, smaller one must not see its leftovers
    for i, (T, d, f) in enumerate((first, second)):
        print(f"[no-alloc] call {i}: T={T} d={d} f={f}", flush=True)
        _both(synthetic.make("decode", T=T, d=d, f=f, seed=900 + T))


def test_static_int8_twice():
    for T in (200, 24):
        w = synthetic.make("int8", T=T, d=256, f=512, seed=950 + T)
        w.scales = synthetic.random_scales(w.E, w.d, w.f, seed=T)
        _both(w)


def test_static_refuses_oversized_shapes():
    w = synthetic.make("decode", T=4096, d=256, f=4096, seed=3)
    assert gm.grok_moe_workspace_bytes(w.T, w.d, w.f, w.E, w.k) > gm.STATIC_WORKSPACE_BYTES
    dev = dev_workload(w, torch)
    out = torch.full_like(dev["x"], 7.0)
    with pytest.raises(gm.GrokMoeError) as ei:
        gm.grok_moe_forward_static(dev["x"], dev["router_w"], dev["w_gate"], dev["w_up"], dev["w_down"], k=w.k,
                                   out=out)
    assert ei.value.code == gm.EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
