"""The seeded input generator: determinism, distributions and a golden digest."""
import json
import math
import os
import sys

import numpy as np

import synthetic

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_golden  # noqa: E402


def test_deterministic_and_thread_independent(monkeypatch):
    a = synthetic.normal((1000, 37), 0, 2, 0.5, "bf16")
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    b = synthetic.normal((1000, 37), 0, 2, 0.5, "bf16")
    np.testing.assert_array_equal(a, b)
    c = synthetic.normal((1000, 37), 1, 2, 0.5, "bf16")
    assert np.mean(a != c) > 0.9


def test_bf16_is_rne_of_f32():
    a32 = synthetic.normal((4097,), 4, 3, 0.1, "f32")
    a16 = synthetic.normal((4097,), 4, 3, 0.1, "bf16")
    np.testing.assert_array_equal(a16, synthetic.f32_to_bf16_bits(a32))


def test_normal_moments():
    z = synthetic.normal((1 << 20,), 0, 9, 1.0, "f32").astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    w = synthetic.normal((1 << 18,), 0, 9, 1 / math.sqrt(6144), "bf16")
    s = synthetic.bf16_bits_to_f32(w).astype(np.float64).std() * math.sqrt(6144)
    assert abs(s - 1) < 1e-2


def test_int8_uniform_range():
    q = synthetic.uniform_i8((1 << 20,), 0, 2)
    assert q.min() == -127 and q.max() == 127
    h = np.bincount(q.astype(np.int64) + 127, minlength=255)
    assert h.min() > 0.8 * h.mean() and h.max() < 1.2 * h.mean()


def test_workload_shapes_and_layouts():
    w = synthetic.make("int8", T=4, f=64)
    assert w.x.shape == (4, 6144) and w.x.dtype == np.uint16
    assert w.router_w.shape == (8, 6144)
    assert w.w_gate.shape == (8, 64, 6144) and w.w_gate.dtype == np.int8
    assert w.w_down.shape == (8, 6144, 64)
    assert w.scales.shape == (2 * 8 * 64 + 8 * 6144,)
    assert np.allclose(w.scales[:8 * 64], 1 / (127 * math.sqrt(6144)))
    assert np.allclose(w.scales[-1], 1 / (127 * math.sqrt(64)))


def test_skew_construction_is_exact():
    w = synthetic.make("skew", T=4, f=64)
    xs = synthetic.bf16_bits_to_f32(w.x[:, -1])
    rs = synthetic.bf16_bits_to_f32(w.router_w[:, -1])
    assert np.all(xs == 1.0)
    assert list(rs) == [3.0, 1.5, 0, 0, 0, 0, 0, 0]


def test_golden_digests():
    ref = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "synthetic_sha256.json")))["digests"]
    assert make_golden.digests() == ref
