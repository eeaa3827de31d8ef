"""The GPU's GELU evaluates Phi(-|z|) with the normal-tail approximation of Abramowitz and Stegun 26.2.17
(after Hastings): Phi(-x) = phi(x) t (b1 + t (b2 + t (b3 + t (b4 + t b5)))), t = 1 / (1 + p x), with a
published absolute error below 7.5e-8. This test reads p, the five coefficients and the exponent constants
out of the kernel header, evaluates the same formula in float32 (as the kernels do, with exact division and
exp2 standing in for v_rcp_f32 and v_exp_f32) and checks it against the fp64 GELU from scipy's erfc, so a
wrong or mistyped constant in the source fails here, on the CPU."""
import os
import re

import numpy as np
import pytest

scipy_special = pytest.importorskip("scipy.special")

HDR = os.path.join(os.path.dirname(__file__), "..", "mixture_experts_transformer_gemm_amd", "csrc", "moe_internal.h")


def _constants():
    src = open(HDR).read()
    body = src[src.index("float gelu_erf(float z)"):]
    body = body[:body.index("\n}\n")]
    p = float(re.search(r"fmaf\(([-0-9.]+)f, fabsf\(z\), 1\.0f\)", body).group(1))
    first = re.search(r"float p = ([-0-9.]+)f;", body).group(1)
    rest = re.findall(r"p = fmaf\(p, t, ([-0-9.]+)f\);", body)
    e2, e0 = re.search(r"fmaf\(z \* z, ([-0-9.]+)f, ([-0-9.]+)f\)", body).groups()
    return p, [float(first)] + [float(c) for c in rest], float(e2), float(e0)


def _gelu_fit_f32(z):
    f = np.float32
    z = z.astype(f)
    p, b, e2, e0 = _constants()
    t = (f(1) / (f(p) * np.abs(z) + f(1))).astype(f)
    poly = np.full_like(z, f(b[0]))
    for c in b[1:]:
        poly = (poly * t + f(c)).astype(f)
    arg = ((z * z).astype(f) * f(e2) + f(e0)).astype(f)
    phi = np.exp2(arg.astype(np.float64)).astype(f)
    q = ((t * poly).astype(f) * phi).astype(f)
    return np.where(z >= 0, z * (f(1) - q), z * q).astype(f)


def test_constants_are_the_published_ones():
    p, b, e2, e0 = _constants()
    # Abramowitz and Stegun 26.2.17: p and b1 .. b5 (the header lists b5 first, Horner order)
    assert p == pytest.approx(0.2316419, abs=1e-9)
    assert b == pytest.approx([1.330274429, -1.821255978, 1.781477937, -0.356563782, 0.319381530], abs=1e-9)
    # phi(z) = 2^(e2 z^2 + e0): e2 = -log2(e) / 2, e0 = -log2(sqrt(2 pi))
    assert e2 == pytest.approx(-0.5 / np.log(2.0), rel=1e-12)
    assert e0 == pytest.approx(-0.5 * np.log2(2.0 * np.pi), rel=1e-12)


def test_gelu_fit_against_exact_erfc():
    z = np.linspace(-14.0, 14.0, 560001).astype(np.float32)
    got = _gelu_fit_f32(z).astype(np.float64)
    zd = z.astype(np.float64)
    ref = 0.5 * zd * scipy_special.erfc(-zd / np.sqrt(2.0))
    err = np.abs(got - ref)
    # the published 7.5e-8 on Phi, times |z|, plus float32 evaluation
    assert (err / np.maximum(1.0, np.abs(zd))).max() <= 3e-7
    pos = zd > 0
    assert (err[pos] / np.abs(ref[pos])).max() <= 1e-6
    # where the far negative tail's values are above the absolute bound, within a bf16 step of them
    neg = (zd < 0) & (np.abs(ref) > 1e-6)
    assert (err[neg] / np.abs(ref[neg])).max() <= 2e-3


def test_gelu_fit_tails_and_zero():
    z = np.array([0.0, -0.0, 30.0, -30.0, 1e-20, -1e-20], dtype=np.float32)
    g = _gelu_fit_f32(z)
    assert g[0] == 0.0 and g[2] == np.float32(30.0) and g[3] == 0.0
    assert g[4] == pytest.approx(0.5e-20, rel=1e-6) and g[5] == pytest.approx(-0.5e-20, rel=1e-6)


def test_gelu_fit_catches_a_wrong_coefficient(monkeypatch):
    """A plausible typo (one coefficient's sign) must break the accuracy check above."""
    p, b, e2, e0 = _constants()
    bad = list(b)
    bad[2] = -bad[2]
    monkeypatch.setattr(__import__(__name__), "_constants", lambda: (p, bad, e2, e0))
    z = np.linspace(-6.0, 6.0, 10001).astype(np.float32)
    got = _gelu_fit_f32(z).astype(np.float64)
    zd = z.astype(np.float64)
    ref = 0.5 * zd * scipy_special.erfc(-zd / np.sqrt(2.0))
    assert (np.abs(got - ref) / np.maximum(1.0, np.abs(zd))).max() > 1e-3
