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
    it was taken on the same workload, W layout, output form and GEMM source."""
    sys.path.insert(0, ROOT)
    import bench
    src_hash = bench.kernel_source_hash()
    f = tmp_path / "traffic.txt"
    g = tmp_path / "traffic_cand.txt"
    f.write_text("# comment: 1\nworkload: 27b-head\nw_layout: packed\n"
                 f"kernel_source_sha256_16: {src_hash}\ntraffic_bytes_per_launch: 123456\n")
    g.write_text("workload: 27b-head\nw_layout: packed\noutput: candidates\n"
                 f"kernel_source_sha256_16: {src_hash}\ntraffic_bytes_per_launch: 654321\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILES", [str(f), str(g)])
    assert bench.measured_traffic("27b-head", "packed", "logits") == 123456.0
    assert bench.measured_traffic("27b-head", "packed", "candidates") == 654321.0
    assert bench.measured_traffic("27b-head", "row-major", "logits") is None   # other W layout
    assert bench.measured_traffic("4b-head", "packed", "logits") is None       # other workload
    f.write_text(f.read_text().replace(src_hash, "0" * 16))
    assert bench.measured_traffic("27b-head", "packed", "logits") is None      # kernel changed
    assert bench.measured_traffic("27b-head", "packed", "candidates") == 654321.0
    monkeypatch.setattr(bench, "TRAFFIC_FILES", [str(tmp_path / "missing.txt")])
    assert bench.measured_traffic("27b-head", "packed", "logits") is None


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


def _binding_cases():
    """(name, call) pairs: each call hands one wrong tensor to a binding
    wrapper; everything else is well formed.  CPU tensors: a wrapper that
    checked the device first would raise about the device instead."""
    import torch

    import block_drafting_amd as bd

    f32, i32 = torch.float32, torch.int32
    B, L, V, r, K = 3, 4, 50, 8, 16
    e = lambda *s, dt=f32: torch.zeros(s, dtype=dt)
    tv, ti = e(B, L, K), e(B, L, K, dt=i32)
    U = e(V, r)
    S0, S = e(B, K), e(B, L - 1, K, K)
    tgt = e(B, L + 1, dt=i32)
    pt = e(B, L, dt=i32)
    u = e(B, L)
    M = B * L
    tm = e(M, 1)
    return [
        ("logits", lambda: bd.topk16_tilemax(e(M, V, dt=torch.bfloat16), tm)),
        ("top_val", lambda: bd.topk16_tilemax(e(M, V), tm, top_val=e(M, 8))),
        ("top_idx", lambda: bd.topk16_tilemax(e(M, V), tm, top_idx=e(M, K))),
        ("top_idx", lambda: bd.topk16(e(M, V), top_idx=e(M + 1, K, dt=i32))),
        ("top_val", lambda: bd.logits_topk(e(M, 64, dt=torch.bfloat16),
                                           e(V, 64, dt=torch.bfloat16), top_val=e(M, K + 1))),
        ("top_val", lambda: bd.pair_score(e(B, L, K, dt=torch.bfloat16), ti, None, U, U)),
        ("S0", lambda: bd.path_select(e(B, K + 1), S, ti)),
        ("S", lambda: bd.path_select(S0, e(B, L, K, K), ti)),
        ("path_score", lambda: bd.path_select(S0, S, ti, path_score=e(B + 1))),
        ("path_tok", lambda: bd.verify_greedy(e(B, L), tgt)),
        ("accept_len", lambda: bd.verify_greedy(pt, tgt, accept_len=e(B, dt=i32).view(1, B))),
        ("top_val", lambda: bd.pair_select_verify(e(B, L, K, dt=torch.float64), ti, None, U, U,
                                                  tgt)),
        ("path_slot", lambda: bd.pair_select_verify(tv, ti, None, U, U, tgt,
                                                    path_slot=e(B, L + 1, dt=i32))),
        ("next_tok", lambda: bd.pair_select_verify(tv, ti, None, U, U, tgt, next_tok=e(B))),
        ("q", lambda: bd.pair_sample(tv, ti, None, U, U, u, 1.0, q=e(B, L, 8))),
        ("S0", lambda: bd.path_sample(e(B, 8), S, ti, u, 1.0)),
        ("S", lambda: bd.path_sample(S0, e(B, L - 2, K, K), ti, u, 1.0)),
        ("path_tok", lambda: bd.path_sample(S0, S, ti, u, 1.0, path_tok=e(B, L))),
        ("z", lambda: bd.target_lse(e(B, L + 1, V, dt=torch.bfloat16), 1.0)),
        ("next_tok", lambda: bd.verify_rejection_lazy(pt, pt, e(B, L, K), ti, e(B, L + 1, V),
                                                      1.0, u, e(B), next_tok=e(B + 2, dt=i32))),
    ]


def test_binding_checks_every_tensor_before_the_device():
    cases = _binding_cases()
    for name, call in cases:
        with pytest.raises((ValueError, TypeError)) as ei:
            call()
        msg = str(ei.value)
        assert name in msg and "GPU" not in msg, (name, msg)


def test_bench_parity_gate_passes_the_oracle_and_catches_mistakes():
    """bench.py's gate before timing: the oracle's own outputs pass it; a
    path changed on a decided block, a logit moved past the 1e-3 bar and a
    decided top-16 slot swapped each fail it.  (The CPU-baseline leg runs
    the oracle; the gate only compares.)"""
    sys.path.insert(0, ROOT)
    import bench
    import oracle as O

    w = WL.WORKLOADS[0]
    inp = WL.make_inputs(w)
    front = O.run_step_front(w, inp)
    targets = WL.make_targets(w, front["top_idx"], front["path_tok"])
    rec, ora = bench.cpu_baseline(w, inp, targets, 1, 1)
    assert rec["cores"] >= 1 and rec["single_core"]["cores"] == 1
    blocks = np.arange(1)
    args = dict(z_rows=ora["z"].copy(), top_val=ora["top_val"].copy(),
                top_idx=ora["top_idx"].copy(), S0=ora["S0"].copy(), S=ora["S"].copy(),
                slot=ora["path_slot"].copy(), accept_len=ora["accept_len"].copy())
    bad, checked = bench.parity_gate(w, blocks, ora, **args)
    assert bad == [] and checked == (1 if ora["margin"][0] > 1e-3 else 0)
    if checked:
        wrong = dict(args, slot=(args["slot"] + 1) % 16)
        assert any("path" in b for b in bench.parity_gate(w, blocks, ora, **wrong)[0])
    z = args["z_rows"].copy()
    z[3, 7] += np.float32(0.01 * max(1.0, abs(float(z[3, 7]))))
    assert any("logits" in b for b in bench.parity_gate(w, blocks, ora, **dict(args, z_rows=z))[0])
    ti = args["top_idx"].copy()
    dec = np.argwhere(ora["gaps"][0] > 1e-3)
    t, s = dec[0]
    ti[0, t, s] = (ti[0, t, s] + 1) % w.V
    assert any("top-16" in b for b in bench.parity_gate(w, blocks, ora, **dict(args, top_idx=ti))[0])
