"""Host-side checks that need no GPU: the benchmark's refusals and the seeded
input generators (thread-count independence, determinism, per-block noise)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_bench_has_no_cpu_fallback():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "needs a GPU" in (r.stdout + r.stderr)


def test_bench_reports_traffic_only_for_the_measured_kernel(tmp_path, monkeypatch):
    """The roofline's traffic comes from a committed counter summary only when
    it was taken on the same workload, W layout and GEMM source."""
    sys.path.insert(0, ROOT)
    import bench
    src_hash = bench.kernel_source_hash()
    f = tmp_path / "traffic.txt"
    f.write_text("# comment: 1\nworkload: 27b-head\nw_layout: packed\n"
                 f"kernel_source_sha256_16: {src_hash}\ntraffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("27b-head", "packed") == 123456.0
    assert bench.measured_traffic("27b-head", "row-major") is None      # other W layout
    assert bench.measured_traffic("4b-head", "packed") is None          # other workload
    f.write_text(f.read_text().replace(src_hash, "0" * 16))
    assert bench.measured_traffic("27b-head", "packed") is None          # kernel changed since
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("27b-head", "packed") is None


def test_chunked_fill_does_not_depend_on_thread_count(monkeypatch):
    n = 3 << 20                                   # above the chunking threshold
    monkeypatch.setattr(WL, "_threads", lambda: 1)
    a = WL.normal_f32((n,), 0.5, 123, WL.TAG_X)
    monkeypatch.setattr(WL, "_threads", lambda: 8)
    b = WL.normal_f32((n,), 0.5, 123, WL.TAG_X)
    np.testing.assert_array_equal(a, b)
    assert abs(float(a.std()) - np.sqrt(0.5)) < 1e-2


def test_tiny_inputs_are_deterministic():
    w = WL.WORKLOADS[0]
    a, b = WL.make_inputs(w), WL.make_inputs(w)
    assert a.keys() == b.keys()
    for k in a:
        if isinstance(a[k], np.ndarray):
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_target_noise_is_per_block():
    w = WL.WORKLOADS[7]
    g = np.random.default_rng(3)
    ti = np.stack([np.stack([g.choice(w.V, 16, replace=False) for _ in range(w.L)])
                   for _ in range(4)]).astype(np.int32)
    full = WL.planted_target_logits(w, ti, np.array([10, 11, 12, 13]))
    sub = WL.planted_target_logits(w, ti[[1, 3]], np.array([11, 13]))
    # the N(0, 1) noise of a block does not depend on which other blocks are drawn
    # (the planted token may differ; compare away from every planted entry)
    for i, j in ((0, 1), (1, 3)):
        mask = np.abs(full[j] - sub[i]) < 1e-6
        assert mask.mean() > 0.999
        diff = ~mask
        assert np.allclose(np.abs(full[j] - sub[i])[diff], WL.TARGET_BUMP, atol=1e-3)


def test_hold_last_extends_profiles():
    np.testing.assert_array_equal(WL.hold_last([0.9, 0.8], 4), [0.9, 0.8, 0.8, 0.8])
    np.testing.assert_array_equal(WL.hold_last([0.9, 0.8, 0.7], 2), [0.9, 0.8])
