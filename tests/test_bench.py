"""Host logic of bench.py (CPU only): the pages' ratio, the roofline bound, the
backward's algorithmic bytes, the profile-hash gate on the traffic figure, and the
single-GPU refusal."""
import os
import subprocess
import sys

import bench
import workloads
from conftest import ROOT


def test_pages_ratio_only_on_the_pages_batch():
    w2 = workloads.make_config(2, with_values=False)
    # The pages' 0.111 ms for 6823 tokens is 61.47 M tokens/s: a tokens/s equal to
    # that gives a ratio of exactly 1.
    assert abs(bench.pages_ratio(w2, 6823 / 0.111e-3) - 1.0) < 1e-12
    assert abs(bench.pages_ratio(w2, 2 * 6823 / 0.111e-3) - 2.0) < 1e-12
    for idx in (1, 3, 4, 5):
        assert bench.pages_ratio(workloads.make_config(idx, with_values=False), 1e9) is None


def test_roofline_bound_follows_the_ridge():
    # config 2: 48.5 FLOP/B, below the ridge: bandwidth against 8 TB/s
    r = bench.roofline(1.355e9, 27.9e6, 10e-6, None, "k")
    assert r["bound"] == "hbm" and abs(r["achieved"] - 2790.0) < 1e-6 and abs(r["frac"] - 2790.0 / 8000.0) < 1e-12
    # config 4: 665 FLOP/B, above it: TFLOP/s against 2500
    r = bench.roofline(69.53e9, 104.5e6, 100e-6, 5.0, "k")
    assert r["bound"] == "mfma" and abs(r["achieved"] - 695.3) < 1e-6 and r["traffic"] == 5.0


def test_backward_algorithmic_bytes():
    w = workloads.make_config(2, with_values=False)
    # 3 KB qkv + 1 KB out + 1 KB dout + 3 KB dqkv + 32 B lse per token (8 heads)
    assert bench.backward_algorithmic_bytes(w) == 6823 * (8 * 1024 + 32)


def test_traffic_needs_profiles_of_the_current_kernel(tmp_path, monkeypatch):
    name = "pages_6823tok_60users"
    prof = tmp_path / "profiles"
    prof.mkdir()
    path = prof / f"attention_kernel_{name}_pmc.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path.write_text(f"# header\nkernel_source_sha256_16: {bench.kernel_source_hash()}\nhbm_bytes_per_launch: 1234.0\n")
    assert bench.kernel_source_hash("bwd") != bench.kernel_source_hash("fwd")
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


def test_visible_pairs_of_the_mask_recipe():
    import numpy as np

    import oracle
    # counted against the oracle's dense mask on a few users (the oracle is test infrastructure)
    lengths, c, g = [5, 40, 1, 0, 300], [2, 16, 1, 0, 9], [1, 30, 0, 0, 32]
    want = sum(int(oracle.hstu_mask(L, min(cc, L), min(gg, L - min(cc, L)), 8, (256, 0)).sum())
               for L, cc, gg in zip(lengths, c, g) if L > 0)
    assert bench.visible_pairs(lengths, c, g, 8, (256, 0)) == want
    # no context, no candidates, no window bound: the causal triangle
    assert bench.visible_pairs([10, 7], [0, 0], [0, 0], 1, (-1, 0)) == 55 + 28
