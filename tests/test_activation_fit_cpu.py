"""The GPU's GELU evaluates Phi(-|z|) = erfc(|z|/sqrt 2)/2 with the Chebyshev fit of Numerical Recipes
(Press et al., 2nd ed., section 6.2, erfcc; published fractional error below 1.2e-7). This test reads the
ten coefficients out of the kernel header, evaluates the same formula in float32 (as the kernels do, with
exact division and exp standing in for v_rcp_f32 and v_exp_f32) and checks it against the fp64 GELU from
scipy's erfc, so a wrong or mistyped constant in the source fails here, on the CPU."""
import os
import re

import numpy as np
import pytest

scipy_special = pytest.importorskip("scipy.special")

HDR = os.path.join(os.path.dirname(__file__), "..", "mixture_experts_transformer_gemm_amd", "csrc", "moe_internal.h")


def _coefficients():
    src = open(HDR).read()
    body = src[src.index("float gelu_erf(float z)"):]
    body = body[:body.index("\n}\n")]
    first = re.search(r"float p = ([-0-9.]+)f;", body).group(1)
    rest = re.findall(r"p = fmaf\(p, t, ([-0-9.]+)f\);", body)
    return [float(first)] + [float(c) for c in rest]


def _gelu_fit_f32(z):
    f = np.float32
    z = z.astype(f)
    u = (np.abs(z) * f(0.70710678118654752)).astype(f)
    t = (f(2) / (f(2) + u)).astype(f)
    c = _coefficients()
    p = np.full_like(u, f(c[0]))
    for ci in c[1:]:
        p = (p * t + f(ci)).astype(f)
    q = (f(0.5) * t * np.exp((p - u * u).astype(np.float64)).astype(f)).astype(f)
    return np.where(z >= 0, z * (f(1) - q), z * q).astype(f)


def test_coefficients_are_the_published_ten():
    c = _coefficients()
    assert len(c) == 10
    # the fit's constant term and leading coefficient (Numerical Recipes erfcc)
    assert c[-1] == pytest.approx(-1.26551223) and c[0] == pytest.approx(0.17087277)


def test_gelu_fit_against_exact_erfc():
    z = np.linspace(-12.0, 12.0, 480001).astype(np.float32)
    got = _gelu_fit_f32(z).astype(np.float64)
    zd = z.astype(np.float64)
    ref = 0.5 * zd * scipy_special.erfc(-zd / np.sqrt(2.0))
    assert np.max(np.abs(got - ref)) <= 5e-7
    nz = np.abs(ref) > 1e-30
    rel = np.abs(got[nz] - ref[nz]) / np.abs(ref[nz])
    assert rel.max() <= 2e-5
    core = nz & (np.abs(zd) <= 4.0)
    assert (np.abs(got[core] - ref[core]) / np.abs(ref[core])).max() <= 3e-6


def test_gelu_fit_tails_and_zero():
    z = np.array([0.0, -0.0, 30.0, -30.0, 1e-20, -1e-20], dtype=np.float32)
    g = _gelu_fit_f32(z)
    assert g[0] == 0.0 and g[2] == np.float32(30.0) and g[3] == 0.0
    assert g[4] == pytest.approx(0.5e-20, rel=1e-6) and g[5] == pytest.approx(-0.5e-20, rel=1e-6)
