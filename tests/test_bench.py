"""Host logic of bench.py (CPU only): the baseline ratio, the profile-hash gate on
the traffic figure, and the single-GPU refusal."""
import os
import subprocess
import sys

import bench
import workloads
from conftest import ROOT


def test_vs_baseline_only_on_the_pages_batch():
    w2 = workloads.make_config(2, with_values=False)
    # The pages' 0.111 ms for 6823 tokens is 61.47 M tokens/s: a tokens/s equal to
    # that gives a ratio of exactly 1.
    assert abs(bench.vs_baseline(w2, 6823 / 0.111e-3) - 1.0) < 1e-12
    assert abs(bench.vs_baseline(w2, 2 * 6823 / 0.111e-3) - 2.0) < 1e-12
    for idx in (1, 3, 4, 5):
        assert bench.vs_baseline(workloads.make_config(idx, with_values=False), 1e9) is None


def test_traffic_needs_profiles_of_the_current_kernel(tmp_path, monkeypatch):
    name = "pages_6823tok_60users"
    prof = tmp_path / "profiles"
    prof.mkdir()
    path = prof / f"attention_kernel_{name}_pmc.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path.write_text(f"# header\nkernel_source_sha256_16: {bench.kernel_source_hash()}\nhbm_bytes_per_launch: 1234.0\n")
    assert bench.measured_traffic(name) == 1234.0
    path.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1234.0\n")
    assert bench.measured_traffic(name) is None
    path.unlink()
    assert bench.measured_traffic(name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
