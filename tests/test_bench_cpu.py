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
