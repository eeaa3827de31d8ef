"""Host-side checks of bench.py: the one-GPU guard and the HBM-traffic lookup
(no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_metric_is_the_headline_string():
    assert bench.METRIC.startswith("MoE-layer tokens/s")


def test_traffic_lookup_checks_the_kernel_sources(tmp_path, monkeypatch):
    files = ["moe_stream.hip", "moe_api.hip", "moe_device.h", "moe_internal.h"]
    good = bench._source_digest(files)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_traffic.txt").write_text(
        "# header\n"
        f"workload=wl_a kernel=k sources={','.join(files)} sha256={good} fetch_kib=100.0 write_kib=10.0 "
        "fetch_factor=2.0 write_factor=1.0\n"
        f"workload=wl_b kernel=k sources={','.join(files)} sha256=0000000000000000 fetch_kib=1 write_kib=1 "
        "fetch_factor=2.0 write_factor=1.0\n")
    # the summary is read from ROOT/profiles; the digest of the listed sources is the repository's own
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_source_digest", lambda fs: good if fs == files else "x")
    assert bench.measured_traffic("wl_a") == (round((100.0 * 2.0 + 10.0) * 1024), "profiles/hbm_traffic.txt")
    assert bench.measured_traffic("wl_b")[0] is None
    assert bench.measured_traffic("wl_c") == (None, "no counter summary for this workload")


@pytest.mark.parametrize("wl", sorted(bench.WORKLOAD_NAMES))
def test_every_bench_workload_has_a_generator_entry(wl):
    import synthetic
    assert wl in synthetic.WORKLOADS


def test_oracle_sample_covers_every_expert():
    # the CPU baseline's sample for large batches: n distinct tokens, at least 8 of every expert with rows
    import numpy as np
    rng = np.random.default_rng(5)
    T, E, k = 3000, 8, 2
    keys = rng.random((T, E)) * (1.0 + 5.0 * (np.arange(E) < 2))     # skewed toward experts 0 and 1
    idx = np.argsort(-keys, axis=1)[:, :k]
    idx[:3] = [[6, 7], [7, 5], [5, 6]]                                 # experts 5..7 get few tokens
    order = np.lexsort((np.repeat(np.arange(T), k), idx.ravel()))
    perm = np.repeat(np.arange(T), k)[order]
    counts = np.bincount(idx.ravel(), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    s = bench.oracle_sample(perm, offsets, T, n=256, per_expert=8, seed=0)
    assert len(s) == 256 and len(np.unique(s)) == 256 and s.min() >= 0 and s.max() < T
    for e in range(E):
        have = np.isin(s, perm[offsets[e]:offsets[e + 1]]).sum()
        assert have >= min(8, counts[e]), (e, have)
    assert np.array_equal(s, bench.oracle_sample(perm, offsets, T, n=256, per_expert=8, seed=0))


def test_expert_split_divides_by_row_tiles():
    # the skewed 2048-token routing at 256-row tiles: 19 row tiles, the cold experts one each
    counts = [1958, 1247, 146, 152, 136, 163, 143, 151]
    s = bench.expert_split(counts, 256, 4.75)
    assert s["tile_rows"] == 256
    tiles = [e["row_tiles"] for e in s["experts"]]
    assert tiles == [8, 5, 1, 1, 1, 1, 1, 1]
    assert [e["empty_rows"] for e in s["experts"]] == [90, 33, 110, 104, 120, 93, 113, 105]
    assert sum(e["gemm_ms"] for e in s["experts"]) == pytest.approx(4.75, abs=1e-3)
    assert s["experts"][0]["gemm_ms"] == pytest.approx(4.75 * 8 / 19, abs=1e-4)
    # an expert without rows runs no tile; no row tiles at all (fp32 path) gives no split
    z = bench.expert_split([0, 300], 128, 1.0)
    assert [e["row_tiles"] for e in z["experts"]] == [0, 3] and z["experts"][0]["gemm_ms"] == 0.0
    assert bench.expert_split([5, 5], 0, 1.0) is None
