#!/usr/bin/env python3
"""Benchmark of the DFlash 2 draft-select-verify step on one MI355X.

One step = one pass of the whole hot path over one batch:
  two-tap conv(s) -> LM-head logits -> top-16 -> [context gate] -> pair
  scores -> path walk (max-plus, or greedy with --walk greedy / the gated
  workload) -> greedy verification,
each stage a call into libdflash2 on the current HIP stream.  Scores, walk
and greedy verification run as one fused launch; a sampled walk runs scores
and walk as one launch, then a rejection verification that computes the
target rows' log-sum-exp itself: every block's first two rows summed up
front, all blocks at once, further rows only where its test reaches them
(--rejection lazy: every row only where the test reaches it; --separate:
scores, walk and verification as separate launches, and for a
sampled walk an lse pass over every target row before the verification).  Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Order of a run:
  1. inputs; a bf16 LM-head weight is packed once into the GEMM's tile
     layout (--row-major-w: read as given); one untimed step gives the
     candidates the verification targets are planted on;
  2. the CPU-baseline leg: the CPU oracle on a bounded block sample, all
     cores of the affinity mask that the BLAS pool may use, then a smaller
     sample on one core; its outputs are the parity gate's reference: the
     GPU's first step must match them under the step's margin rules, else
     the run exits with status 3 before any timing (--no-cpu-baseline
     skips both);
  3. W warmup steps, then replays of the captured step until the clocks have
     run for at least --settle seconds (the GPU ramps its clock over the
     first few hundred milliseconds of load);
  4. the timed region: the K steps captured as one HIP graph and replayed
     once (--eager: K plain launches); then the stage pass: half a settle
     period of replays and K eager steps with HIP events between the stages
     (the GEMM's events bracket its one launch), enqueued without a
     synchronisation in between.

Prints ONE JSON line (rank 0, N = 1):
  value = blocks/s over the timed steps (B / seconds per step);
  roofline = the LM-head GEMM kernel (the dominant kernel) against the bf16
  matrix-core peak (against HBM when its flop per algorithmic byte is below
  the ridge, as for the 4b-head workload), its duration the mean of its
  events over the stage pass, which follows the timed region at the same
  sustained load;
  stage_ms = per-stage times from the stage pass;
  accept_len = mean acceptance of the step's path, and of the top-1 path and
  the oracle selector on the same planted targets (greedy verification);
  cpu_baseline = the CPU oracle on the block sample, same inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector peak (fp32 workload)
PEAK_HBM_GBS = 8000.0
# counter summaries of the GEMM: logits written, and the candidate form
TRAFFIC_FILES = [os.path.join(ROOT, "profiles", f) for f in
                 ("lmhead_gemm_27b_head_traffic.txt", "lmhead_candidates_27b_head_traffic.txt")]
PEAKS_FILE = os.path.join(ROOT, "profiles", "peaks_mfma_hbm.txt")


def measured_peaks():
    """The attainable peaks measured on this part (profiles/peaks_mfma_hbm.txt:
    bench.py --peaks), or {} when the summary is missing."""
    out = {}
    if os.path.exists(PEAKS_FILE):
        for line in open(PEAKS_FILE):
            m = re.match(r"^([a-z0-9_]+):\s*([0-9.]+)\s*$", line)
            if m:
                out[m.group(1)] = float(m.group(2))
    return out


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[0, 1, 2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--walk", choices=["viterbi", "greedy"], default=None,
                    help="path walk (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU-baseline leg and with it the parity gate")
    ap.add_argument("--cpu-blocks", type=int, default=64,
                    help="blocks the CPU oracle runs on all cores (also the parity sample)")
    ap.add_argument("--cpu-blocks-single", type=int, default=8,
                    help="blocks the CPU oracle runs on one core")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of step replays after the warmup steps, before timing")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--peaks", action="store_true",
                    help="measure attainable peaks (matrix-core probe, HBM copy) and exit")
    ap.add_argument("--sweep", choices=["topk", "pair"], default=None,
                    help="scaled-batch sweep of the top-16 or the fused pair + walk + verify; "
                         "one JSON line per size, then exit")
    ap.add_argument("--sweep-sizes", default=None,
                    help="comma-separated rows (topk) or blocks (pair) for --sweep")
    ap.add_argument("--gemm-vs-vendor", type=int, default=None, metavar="M",
                    help="time the LM-head GEMM (logits form and candidate form, W packed) "
                         "beside the vendor GEMM (torch.mm: hipBLASLt) at M rows of the 27b-head "
                         "shape (K = 5120, N = 151936), one JSON line, then exit")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--separate", action="store_true",
                    help="pair scores, walk and verification as separate launches, and for a "
                         "sampled walk the lse pass over every target row before the "
                         "verification (default: fused scores + walk, lazy verification)")
    ap.add_argument("--row-major-w", action="store_true",
                    help="LM-head GEMM reads W [V, H] as given (default for bf16: W packed once, "
                         "before timing, into the GEMM's 256 x 64 tile layout)")
    ap.add_argument("--keep-logits", action="store_true",
                    help="write all [M, V] logits (default for bf16: the GEMM's candidate form, "
                         "which writes only the tiles and values the top-16 may need)")
    ap.add_argument("--rejection", choices=["staged", "lazy"], default="staged",
                    help="sampled walks: the lazy verification with every block's first two "
                         "target rows summed up front (staged, default) or each row read "
                         "only when the accept test reaches it (lazy); the same results")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of the captured step")
    return ap.parse_args(argv)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "block_drafting_amd", "csrc", "lmhead.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str, w_layout: str, form: str):
    """HBM bytes per GEMM launch from a committed counter summary, if one was
    taken on this workload, W layout and output form ("logits" or
    "candidates") with the current kernel source; else None."""
    for path in TRAFFIC_FILES:
        if not os.path.exists(path):
            continue
        kv = {}
        for line in open(path):
            m = re.match(r"^\s*([a-z0-9_]+)\s*[:=]\s*(\S+)", line)
            if m:
                kv[m.group(1)] = m.group(2)
        if (kv.get("kernel_source_sha256_16") == kernel_source_hash()
                and kv.get("workload") == workload and kv.get("w_layout") == w_layout
                and kv.get("output", "logits") == form):
            try:
                return float(kv["traffic_bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def _time_events(fn, reps: int, settle_s: float = 0.3):
    """Median milliseconds of fn() over reps launches, each bracketed by
    events on the current stream, after settle_s seconds of launches."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        fn()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2]


def peaks():
    """Attainable peaks on this GPU, measured: the GEMM's matrix-core work
    without memory traffic (the library's probe: 256 workgroups of eight
    waves, v_mfma_f32_32x32x16_bf16 on register operands) with operands of
    the benchmark's bit statistics (N(0, 1) in bf16) and with zeros, and a
    plain 4 GiB device copy (above the 256 MB MALL)."""
    import torch
    import block_drafting_amd as bd
    nwg, iters = 256, 20000
    flops = nwg * 8 * iters * 8 * 2 * 32 * 32 * 16
    nbytes = bd.probe_mfma_operand_bytes(nwg)
    rnd = torch.randn(nbytes // 2, device="cuda").to(torch.bfloat16)
    zero = torch.zeros(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(nwg * 512, device="cuda")
    for name, ops in (("normal", rnd), ("zeros", zero)):
        ms = _time_events(lambda: bd.probe_mfma(ops, nwg, iters, out), 7, settle_s=1.0)
        print(json.dumps({"peak": "mfma_bf16", "operands": name, "workgroups": nwg,
                          "iters": iters, "ms": round(ms, 4),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}), flush=True)
    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    ms = _time_events(lambda: b.copy_(a), 7, settle_s=1.0)
    print(json.dumps({"peak": "hbm_copy", "bytes_read": n, "bytes_written": n,
                      "ms": round(ms, 4), "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def gemm_vs_vendor(M: int):
    """The LM-head GEMM beside the vendor GEMM at M rows of the 27b-head
    shape (K = 5120, N = 151936, bf16 operands of the benchmark's
    statistics): ours writing the fp32 logits (dflash2_lmhead_logits, W
    packed) and in the candidate form (dflash2_logits_topk without a logits
    buffer: the group-maxima reset, the GEMM and the top-16 merge), and
    torch.mm (hipBLASLt) with bf16 and with fp32 output.  Medians of 10
    event-timed calls after 0.5 s of calls each."""
    import torch
    import block_drafting_amd as bd
    H, V = 5120, 151936
    g = torch.Generator(device="cuda").manual_seed(3)
    h = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    Wp = bd.lmhead_pack(W)
    Wt = W.t()
    z = torch.empty((M, V), device="cuda")
    o16 = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(bd.logits_topk_workspace(M, H, V, torch.bfloat16, False), dtype=torch.uint8,
                     device="cuda")
    tv = torch.empty((M, 16), device="cuda")
    ti = torch.empty((M, 16), dtype=torch.int32, device="cuda")
    fns = {"lmhead_logits": lambda: bd.lmhead_logits(h, Wp, z),
           "logits_topk_candidates": lambda: bd.logits_topk(h, Wp, top_val=tv, top_idx=ti,
                                                            workspace=ws),
           "torch_mm_bf16_out": lambda: torch.mm(h, Wt, out=o16),
           "torch_mm_f32_out": lambda: torch.mm(h, Wt, out_dtype=torch.float32)}
    rec = {"gemm_vs_vendor": {"M": M, "K": H, "N": V}}
    for name, fn in fns.items():
        us = _time_events(fn, 10, settle_s=0.5) * 1e3
        rec[name] = {"us": round(us, 1), "tflops": round(2 * M * H * V / (us * 1e-6) / 1e12, 1)}
    print(json.dumps(rec), flush=True)


def sweep(kind: str, sizes):
    """Scaled-batch sweep of the small stages, synthetic inputs of the
    27b-head shapes, one JSON line per size (median of 7 timed launches
    after 0.3 s of launches).

    topk: rows M of N(0, 1) fp32 logits over V = 151936 tokens and their
      256-column tile maxima; the pruned top-16 (dflash2_topk16_tilemax) and
      the full scan (dflash2_topk16).  Algorithmic bytes: the full scan reads
      M V 4; the pruned one reads the tile maxima and at least the 16 tiles
      that hold the top-16, M (ceil(V / 256) 4 + 16 1024).
    pair: B blocks of L = 8 random candidates (ids uniform over V), bf16
      factor tables [V, 64], random targets; the fused scores + max-plus walk
      + greedy verification (dflash2_pair_select_verify).  Algorithmic bytes
      per block: the factor rows gathered, 2 L 16 r 2, the candidates,
      L 16 8, the targets and the outputs, (4 L + 3) 4."""
    import torch
    import block_drafting_amd as bd
    g = torch.Generator(device="cuda").manual_seed(7)
    V = 151936
    if kind == "topk":
        nt = (V + 255) // 256
        for M in sizes:
            z = torch.randn((M, V), generator=g, device="cuda")
            tm = torch.empty((M, nt), device="cuda")
            for r0 in range(0, M, 4096):          # tile maxima, a band of rows at a time
                zz = z[r0:r0 + 4096]
                zp = torch.nn.functional.pad(zz, (0, nt * 256 - V), value=float("-inf"))
                tm[r0:r0 + 4096] = zp.view(zz.shape[0], nt, 256).amax(dim=2)
                del zp
            tv = torch.empty((M, 16), device="cuda")
            ti = torch.empty((M, 16), dtype=torch.int32, device="cuda")
            ws = torch.empty(max(bd.topk16_workspace(M, V), 1), dtype=torch.uint8, device="cuda")
            ms_p = _time_events(lambda: bd.topk16_tilemax(z, tm, tv, ti), 7)
            ms_f = _time_events(lambda: bd.topk16(z, tv, ti, ws), 7)
            alg_p = M * (nt * 4 + 16 * 1024)
            alg_f = M * V * 4
            print(json.dumps({"sweep": "topk", "rows": M, "V": V,
                              "pruned_us": round(ms_p * 1e3, 1), "pruned_alg_bytes": alg_p,
                              "pruned_gbs": round(alg_p / (ms_p * 1e-3) / 1e9, 1),
                              "scan_us": round(ms_f * 1e3, 1), "scan_bytes": alg_f,
                              "scan_gbs": round(alg_f / (ms_f * 1e-3) / 1e9, 1)}), flush=True)
            del z, tm
            torch.cuda.empty_cache()
    else:
        L, r = 8, 64
        U = (torch.randn((V, r), generator=g, device="cuda") * 0.316).to(torch.bfloat16)
        Vf = (torch.randn((V, r), generator=g, device="cuda") * 0.316).to(torch.bfloat16)
        for B in sizes:
            tv = torch.randn((B, L, 16), generator=g, device="cuda").sort(dim=2, descending=True)[0]
            ti = torch.randint(0, V, (B, L, 16), generator=g, device="cuda", dtype=torch.int32)
            at = torch.randint(0, V, (B,), generator=g, device="cuda", dtype=torch.int32)
            tgt = torch.randint(0, V, (B, L + 1), generator=g, device="cuda", dtype=torch.int32)
            outs = [torch.empty((B, L), dtype=torch.int32, device="cuda"),
                    torch.empty((B, L), dtype=torch.int32, device="cuda"),
                    torch.empty((B,), device="cuda"),
                    torch.empty((B,), dtype=torch.int32, device="cuda"),
                    torch.empty((B,), dtype=torch.int32, device="cuda")]
            ms = _time_events(lambda: bd.pair_select_verify(tv, ti, at, U, Vf, tgt, None,
                                                            "viterbi", None, None, *outs), 7)
            alg = B * (2 * L * 16 * r * 2 + L * 16 * 8 + (4 * L + 3) * 4)
            print(json.dumps({"sweep": "pair_select_verify", "blocks": B, "L": L, "r": r,
                              "us": round(ms * 1e3, 1), "alg_bytes": alg,
                              "gbs": round(alg / (ms * 1e-3) / 1e9, 1)}), flush=True)


def cpu_baseline(w, inp, targets, n_blocks: int, n_single: int):
    """The CPU oracle (test infrastructure) on a bounded block sample.

    The first n_blocks blocks run with the BLAS pool's threads (at most the
    CPUs of the process affinity mask), then the first n_single blocks on
    one thread.  Verification runs against the targets the GPU step uses
    (greedy) or the planted target logits (sampled).  Returns the baseline
    record and the oracle's outputs for the first sample, with the margins
    the parity gate needs (top-16 gaps, the walk's decision margin)."""
    import threadpoolctl
    import oracle as O
    import workloads as WL

    affinity = len(os.sched_getaffinity(0))
    pool = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    threads = max(1, min(affinity, pool))

    def run(blocks):
        ora = O.run_step_front(w, inp, blocks)
        if w.temperature > 0:
            zt = WL.planted_target_logits(w, ora["top_idx"], blocks)
            ora["accept_len"], ora["next_tok"] = O.rejection_verify(
                ora["path_tok"], ora["q"], ora["top_idx"], zt, w.temperature,
                inp["u_acc"][blocks], inp["u_res"][blocks])
        else:
            ora["accept_len"], ora["next_tok"] = O.verify_greedy(ora["path_tok"],
                                                                 targets[blocks])
        return ora

    blocks = np.arange(min(n_blocks, w.B))
    with threadpoolctl.threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        ora = run(blocks)
        dt = time.perf_counter() - t0
    single = np.arange(min(n_single, len(blocks)))
    dt1 = None
    if len(single):
        with threadpoolctl.threadpool_limits(limits=1):
            t0 = time.perf_counter()
            run(single)
            dt1 = time.perf_counter() - t0
    # margins for the parity gate (oracle helpers, computed in this leg)
    ora["gaps"] = O.topk_gaps(ora["z"], ora["top_val"].reshape(-1, 16)).reshape(
        ora["top_idx"].shape)
    if w.walk in ("sample", "sample-path"):
        ora["margin"] = O.sample_margin(ora["q"], inp["u_path"][blocks])
    elif w.walk == "greedy":
        ora["margin"] = O.greedy_margin(ora["S0"], ora["S"], ora["path_slot"])
    else:
        ora["margin"] = O.path_margin(ora["S0"], ora["S"])
    rec = {"value": len(blocks) / dt, "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
           "sample": f"first {len(blocks)} of {w.B} blocks of the {w.name} workload (full conv, "
                     f"logits over all {w.V} tokens, top-16, pairs, path, verify), {dt:.1f} s, "
                     f"fp64 numpy/OpenBLAS on {threads} threads ({affinity} CPUs in the "
                     f"affinity mask)"}
    if dt1 is not None:
        rec["single_core"] = {"value": len(single) / dt1, "unit": "blocks/s", "cores": 1,
                              "sample": f"first {len(single)} blocks, {dt1:.1f} s on one thread"}
    return rec, ora


def parity_gate(w, blocks, ora, z_rows, top_val, top_idx, S0, S, slot, accept_len):
    """The GPU's first step against the oracle on the sample, under the
    step's margin rules (the end-to-end bars of the GPU tests): logits within
    1e-3 max(|z|, 1); a top-16 slot equal where the oracle's gaps to its
    neighbours exceed 1e-3; a path (and its acceptance) equal where the
    oracle's decision margin exceeds 1e-3 plus the score drift.  Returns a
    list of failures (empty when the step passes)."""
    bad = []
    zo = ora["z"].astype(np.float64)
    err = np.abs(z_rows.astype(np.float64) - zo)
    if not np.all(err <= 1e-3 * np.maximum(np.abs(zo), 1.0)):
        bad.append(f"logits: max |dz| {err.max():.3g}")
    decided = ora["gaps"] > 1e-3
    if not np.array_equal(top_idx[decided], ora["top_idx"][decided]):
        bad.append(f"top-16: {(top_idx[decided] != ora['top_idx'][decided]).sum()} decided slots")
    L = ora["top_idx"].shape[1]
    same = (top_idx == ora["top_idx"]).all(axis=(1, 2))
    checked = 0
    for k in range(len(blocks)):
        if not same[k]:
            continue
        drift = np.abs(S0[k] - ora["S0"][k]).max()
        if L > 1:
            drift = max(drift, np.abs(S[k] - ora["S"][k]).max())
        if w.walk == "sample":
            clear = (ora["margin"][k] > 1e-5 + 2 * 16 * drift / w.temperature).all()
        elif w.walk == "sample-path":
            # the fp32 backward messages' error bound, plus the drift
            # carried through L messages
            smax = max(np.abs(ora["S0"][k]).max(), np.abs(ora["S"][k]).max() if L > 1 else 0)
            tol = 8 * 2.0 ** -24 * L * (smax / w.temperature + 4.0)
            clear = (ora["margin"][k] > tol + 2 * 16 * L * drift / w.temperature).all()
        else:
            clear = ora["margin"][k] > 1e-3 + 2 * L * drift
        if not clear:
            continue
        checked += 1
        if slot[k].tolist() != ora["path_slot"][k].tolist():
            bad.append(f"path of block {blocks[k]}")
        elif w.temperature <= 0 and accept_len[k] != ora["accept_len"][k]:
            bad.append(f"acceptance of block {blocks[k]}")
    return bad, checked


def acceptance(path_tok, target):
    """Greedy acceptance lengths: 1 + the leading matches with the targets."""
    L = path_tok.shape[1]
    return np.cumprod(path_tok == target[:, :L], axis=1).sum(axis=1) + 1


def main(argv=None):
    a = parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the step shards by "
              "block with no exchange, so N GPUs would run N independent copies", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if a.copy_calib:
        copy_calibration()
        return 0
    if a.peaks or a.sweep or a.gemm_vs_vendor:
        sys.path.insert(0, ROOT)
        if a.peaks:
            peaks()
        elif a.gemm_vs_vendor:
            gemm_vs_vendor(a.gemm_vs_vendor)
        else:
            default = "512,4096,16384,65536" if a.sweep == "topk" else "64,1024,8192,32768"
            sweep(a.sweep, [int(v) for v in (a.sweep_sizes or default).split(",")])
        return 0

    sys.path.insert(0, ROOT)
    import block_drafting_amd as bd
    import workloads as WL

    w = WL.WORKLOADS[a.workload]
    if a.walk is not None:
        w = w.shrink(walk=a.walk)
    bf16 = w.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    log(f"[bench] workload {w.cid} {w.name}: B={w.B} L={w.L} H={w.H} V={w.V} r={w.r} "
        f"convs={w.n_convs}; generating inputs")
    t0 = time.perf_counter()
    inp = WL.make_inputs(w)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(arr, kind):
        arr = np.ascontiguousarray(arr)
        if kind == "act":
            if bf16:
                return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(arr).cuda()
        return torch.from_numpy(arr).cuda()

    x = dev(inp["x"], "act")
    convs = [{"k0": dev(c["k0"], "f32"), "k1": dev(c["k1"], "f32"), "anchor_h": dev(c["anchor_h"], "act"),
              "proj": None if c["proj"] is None else dev(c["proj"], "f32"), "groups": c["groups"],
              "projT": None if c["projT"] is None else dev(c["projT"], "act")}
             for c in inp["convs"]]
    W = dev(inp["W"], "act")
    packed = bf16 and not a.row_major_w
    w_layout = "packed" if packed else "row-major"
    if packed:
        # a decoding loop re-lays its LM-head weight out once, not per step
        W = bd.lmhead_pack(W)
    U = dev(inp["U"], "act")
    Vf = dev(inp["Vf"], "act")
    anchor = dev(inp["anchor_tok"], "i32")
    Wg = dev(inp["Wg"], "act") if w.gate else None
    B, L, H, V = w.B, w.L, w.H, w.V
    M = B * L
    sampled = w.temperature > 0
    cand_form = bf16 and not a.keep_logits   # GEMM writes candidates, not the logits
    buf = bd.StepBuffers(B, L, H, V, tdt, "cuda", n_convs=w.n_convs, keep_logits=not cand_form,
                         gate_rank=w.r if w.gate else 0, sample=sampled)
    tilemax = (None if cand_form else
               torch.empty((M, (V + bd.TILEMAX_COLS - 1) // bd.TILEMAX_COLS),
                           dtype=torch.float32, device="cuda"))
    if sampled:
        u_path, u_acc, u_res = (dev(inp[k], "f32") for k in ("u_path", "u_acc", "u_res"))

    # one untimed step gives the candidates the verification targets are planted on
    bd.run_step(buf, x, convs, W, U, Vf, anchor, None, Wg=Wg, walk=w.walk,
                temperature=w.temperature, u_path=u_path if sampled else None)
    torch.cuda.synchronize()
    cand = buf.top_idx.view(B, L, 16).cpu().numpy()
    targets = None
    if sampled:
        # the target model's logits for every drafted position (+ the bonus one)
        z_target = torch.from_numpy(WL.planted_target_logits(w, cand)).cuda()
    else:
        targets = WL.make_targets(w, cand, buf.path_tok.cpu().numpy())
        target = torch.from_numpy(targets).cuda()
    first = {"top_val": buf.top_val.view(B, L, 16).cpu().numpy(), "top_idx": cand,
             "S0": buf.S0.cpu().numpy(), "S": buf.S.cpu().numpy(),
             "path_slot": buf.path_slot.cpu().numpy()}

    fused = not a.separate                 # scores + walk (+ greedy verification) in one launch
    two_pass = sampled and a.separate      # lse of every target row, then the verification
    final_y = buf.y[(len(convs) - 1) % len(buf.y)] if convs else x   # the chain's output
    smode = "path" if w.walk == "sample-path" else "chain"
    gate = buf.gate if w.gate else None
    tv3, ti3 = buf.top_val.view(B, L, 16), buf.top_idx.view(B, L, 16)

    def st_conv():
        cur = x
        for j, c in enumerate(convs):
            out = buf.y[j % len(buf.y)]
            if c["projT"] is not None:
                bd.twotap_conv_mm(cur, c["k0"], c["k1"], c["projT"], c["anchor_h"], out=out)
            else:
                bd.twotap_conv(cur, c["k0"], c["k1"], c["anchor_h"], c["proj"], c["groups"], out=out)
            cur = out

    if cand_form:
        stages = [
            ("conv", st_conv),
            ("gemm", lambda: bd.lmhead_candidates(final_y.view(M, H), W, buf.workspace)),
            ("topk", lambda: bd.topk16_candidates(buf.workspace, M, H, V, buf.top_val,
                                                  buf.top_idx)),
        ]
    else:
        stages = [
            ("conv", st_conv),
            ("gemm", lambda: bd.lmhead_logits_tilemax(final_y.view(M, H), W, buf.logits,
                                                      tilemax)),
            ("topk", lambda: bd.topk16_tilemax(buf.logits, tilemax, buf.top_val, buf.top_idx)),
        ]
    if w.gate:
        stages.append(("gate", lambda: bd.context_gate(final_y.view(M, H), Wg, buf.gate)))
    if fused and sampled:
        # scores and the sampling walk in one launch, then the staged (or lazy) verification
        stages += [
            ("pair_sample", lambda: bd.pair_sample(tv3, ti3, anchor, U, Vf, u_path, w.temperature,
                                                   gate, None, None, buf.path_slot,
                                                   buf.path_tok, buf.q, mode=smode)),
            ("verify", (lambda: bd.verify_rejection_staged(
                buf.path_slot, buf.path_tok, buf.q, ti3, z_target, w.temperature, u_acc, u_res,
                buf.accept_len, buf.next_tok, workspace=buf.staged))
             if a.rejection == "staged" else
             (lambda: bd.verify_rejection_lazy(buf.path_slot, buf.path_tok, buf.q, ti3,
                                               z_target, w.temperature, u_acc, u_res,
                                               buf.accept_len, buf.next_tok)))]
    elif fused:
        # scores, walk and verification in one launch; the scores stay on chip
        stages.append(("pair_select_verify", lambda: bd.pair_select_verify(
            tv3, ti3, anchor, U, Vf, target, gate, w.walk, None, None, buf.path_slot,
            buf.path_tok, buf.path_score, buf.accept_len, buf.next_tok)))
    else:
        stages.append(("pair", lambda: bd.pair_score(tv3, ti3, anchor, U, Vf, buf.S0, buf.S,
                                                     gate=gate)))
        if sampled:
            stages += [
                ("select", lambda: bd.path_sample(buf.S0, buf.S, ti3, u_path, w.temperature,
                                                  buf.path_slot, buf.path_tok, buf.q,
                                                  mode=smode)),
                ("lse", lambda: bd.target_lse(z_target, w.temperature, buf.lse)),
                ("verify", lambda: bd.verify_rejection(buf.path_slot, buf.path_tok, buf.q, ti3,
                                                       z_target, buf.lse, w.temperature, u_acc,
                                                       u_res, buf.accept_len, buf.next_tok))]
        else:
            stages += [
                ("select", lambda: bd.path_select(buf.S0, buf.S, ti3, buf.path_slot,
                                                  buf.path_tok, buf.path_score, mode=w.walk)),
                ("verify", lambda: bd.verify_greedy(buf.path_tok, target, buf.accept_len,
                                                    buf.next_tok))]
    order = [k for k, _ in stages]

    def step():
        for _, f in stages:
            f()

    # the first full step (with its verification) for the parity gate
    step()
    torch.cuda.synchronize()
    first["accept_len"] = buf.accept_len.cpu().numpy()

    cpu = None
    if not a.no_cpu_baseline:
        log(f"[bench] CPU-baseline leg: oracle on {min(a.cpu_blocks, B)} blocks "
            f"(all cores), {min(a.cpu_blocks_single, a.cpu_blocks, B)} blocks (one core)")
        cpu, ora = cpu_baseline(w, inp, targets, a.cpu_blocks, a.cpu_blocks_single)
        blocks = np.arange(len(ora["top_idx"]))
        rows = (blocks[:, None] * L + np.arange(L)[None, :]).reshape(-1)
        rows_t = torch.from_numpy(rows).cuda()
        if cand_form:
            # the candidate form keeps no logits: the same GEMM once more, untimed
            z_rows = bd.lmhead_logits(final_y.view(M, H), W)[rows_t].cpu().numpy()
        else:
            z_rows = buf.logits[rows_t].cpu().numpy()
        bad, checked = parity_gate(w, blocks, ora, z_rows, first["top_val"][blocks],
                                   first["top_idx"][blocks], first["S0"][blocks],
                                   first["S"][blocks], first["path_slot"][blocks],
                                   first["accept_len"][blocks])
        if bad:
            log(f"[bench] PARITY GATE FAILED against the oracle: {'; '.join(bad[:8])}")
            return 3
        log(f"[bench] parity gate passed on {len(blocks)} blocks ({checked} paths decided "
            "and compared exactly)")
        cpu["parity_gate"] = {"blocks": int(len(blocks)), "paths_compared": int(checked)}

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    outs = (buf.top_val, buf.top_idx, buf.path_slot, buf.path_tok, buf.accept_len, buf.next_tok)
    eager_out = [t.clone() for t in outs]

    # Each step enqueues on the current stream and allocates nothing, so it
    # can be captured: a one-step graph for the clock settling and the K
    # timed steps as one graph.
    graph1 = graphK = None
    if not a.eager:
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step()
            torch.cuda.synchronize()
            graph1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph1, stream=cap):
                step()
            graphK = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphK, stream=cap):
                for _ in range(a.steps):
                    step()

        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
    one = graph1.replay if graph1 is not None else step
    # clock settling: replays until --settle seconds have passed
    t0 = time.perf_counter()
    settle_steps = 0
    while True:
        for _ in range(16):
            one()
        settle_steps += 16
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= a.settle:
            break
    settle_s = time.perf_counter() - t0
    log(f"[bench] warmup done ({a.warmup} steps, then {settle_steps} steps in {settle_s:.2f} s); "
        f"timing {a.steps} steps ({'one graph of K steps' if graphK is not None else 'eager'})")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if graphK is not None:
        graphK.replay()
    else:
        for _ in range(a.steps):
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] timed {a.steps} steps in {wall:.3f} s")
    for t, r in zip(outs, eager_out):          # the replays computed what eager steps do
        assert torch.equal(t, r), "graph replay differs from the eager step"

    # light sanity on the last step's outputs
    acc = buf.accept_len.cpu().numpy()
    tv = buf.top_val.cpu().numpy()
    assert ((acc >= 1) & (acc <= L + 1)).all() and (np.diff(tv, axis=1) <= 0).all()

    # per-stage times: half a settle period of step replays (the clocks drop
    # while the host checks the timed outputs), then K eager steps with
    # events on the stream between the stages, all enqueued before one
    # synchronisation: the host runs far ahead, so the GPU executes them back
    # to back at the load of the timed region
    ev_all = [{k: torch.cuda.Event(enable_timing=True) for k in order + ["end"]}
              for _ in range(a.steps)]
    for _ in range(max(16, settle_steps // 2)):
        one()
    for i in range(a.steps):
        for k, f in stages:
            ev_all[i][k].record()
            f()
        ev_all[i]["end"].record()
    torch.cuda.synchronize()
    stage_wall_ms = ev_all[0]["conv"].elapsed_time(ev_all[-1]["end"]) / a.steps
    stage_ms = {k: 0.0 for k in order}
    for i in range(a.steps):
        marks = [ev_all[i][k] for k in order] + [ev_all[i]["end"]]
        for k, s_, e_ in zip(order, marks[:-1], marks[1:]):
            stage_ms[k] += s_.elapsed_time(e_) / a.steps
    gemm_ms = [ev_all[i]["gemm"].elapsed_time(ev_all[i]["topk"]) for i in range(a.steps)]
    # per-step times of the stage pass (the timed region is one replay of K
    # steps, so its per-step spread is taken here)
    step_ms = sorted(ev_all[i]["conv"].elapsed_time(ev_all[i]["end"]) for i in range(a.steps))
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(round(q * (len(step_ms) - 1))))]
    ms_step = wall * 1e3 / a.steps
    gemm_s = float(np.mean(gemm_ms)) * 1e-3
    flops = 2.0 * M * H * V
    # algorithmic GEMM bytes: W and h read once, tile maxima written, and the
    # logits (logits form) or the per-tile counts (candidate form)
    nt = (V + 255) // 256
    gemm_bytes = ((V * H + M * H) * (2 if bf16 else 4) + M * nt * 4
                  + (M * nt * 4 if cand_form else M * V * 4))
    form = "candidates" if cand_form else "logits"
    if bf16 and flops / gemm_bytes < PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        # below the ridge (small M): HBM-bound
        achieved = gemm_bytes / gemm_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(w.name, w_layout, form)}
    elif bf16:
        achieved = flops / gemm_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(w.name, w_layout, form)}
    else:
        achieved = flops / gemm_s / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_F32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F32_TFLOPS, 5), "traffic": None}
    pk = measured_peaks()
    if roof["bound"] == "mfma" and "mfma_bf16_attainable_tflops_normal_operands" in pk:
        # the matrix-core rate this part sustains on operands of these
        # statistics (the GEMM's work without memory traffic), as context
        att = pk["mfma_bf16_attainable_tflops_normal_operands"]
        roof["attainable"] = att
        roof["frac_of_attainable"] = round(achieved / att, 4)
    # algorithmic HBM rates of the streaming stages, against 8 TB/s
    es = 2 if bf16 else 4
    conv_bytes = w.n_convs * (2 * L + 1) * B * H * es
    if w.dynamic and w.groups > 1:
        conv_bytes += w.n_convs * 2 * w.groups * H * es      # the correction maps
    hbm = {"conv": round(conv_bytes / (stage_ms["conv"] * 1e-3) / 1e9, 1)}
    if two_pass:
        hbm["lse"] = round(B * (L + 1) * V * 4 / (stage_ms["lse"] * 1e-3) / 1e9, 1)
    # per-stage rooflines: bytes per launch (the basis stated), GB/s and the
    # fraction of 8 TB/s; the top-16 reads the tile maxima and at least the
    # 16 tiles that hold the top-16 (the counters read 1.03x that at this
    # size); the fused pair stage gathers two factor rows per candidate
    basis = {"conv": (conv_bytes, "(2L+1) B H per application: x, predecessors, y"),
             "topk": ((M * (nt * 8 + 16 * 32),
                       "M (ceil(V/256) 8 + 16 x 32): tile maxima, counts, 16 tiles' slots")
                      if cand_form else
                      (M * (nt * 4 + 16 * 1024),
                       "M (ceil(V/256) 4 + 16 KiB): tile maxima + 16 tiles"))}
    if fused and not sampled:
        basis["pair_select_verify"] = (
            B * (2 * L * 16 * w.r * 2 + L * 16 * 8 + (4 * L + 3) * 4),
            "B (2 L 16 r 2 + L 16 8 + (4 L + 3) 4): factor rows, candidates, targets, outputs")
    if fused and sampled:
        # the target rows the verification reads, from this run's acceptance
        # lengths n + 1: the staged form sums the first min(2, L + 1) rows of
        # every block and reads the rows past them that a test reaches; the
        # lazy form reads rows 0 .. n of each block
        n_rows = acc.astype(np.int64)
        if a.rejection == "staged":
            k = min(bd.STAGED_ROWS, L + 1)
            rows_read = B * k + int(np.maximum(n_rows - k, 0).sum())
            why = "V 4 x (B 2 staged rows + the rows past them the tests reach)"
        else:
            rows_read = int(n_rows.sum())
            why = "V 4 x (n + 1 rows of each block, n = tokens accepted)"
        basis["verify"] = (rows_read * V * 4, why)
    stage_roof = {}
    for k, (nb, why) in basis.items():
        gbs = nb / (stage_ms[k] * 1e-3) / 1e9
        stage_roof[k] = {"bytes": int(nb), "basis": why, "gbs": round(gbs, 1),
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}
    accept = {"path": round(float(acc.mean()), 3)}
    if not sampled and w.target_mode != "mix":
        # the same planted targets read by the top-1 path and by the oracle
        # selector (the target's token whenever it is a candidate, else slot 0)
        ti = buf.top_idx.view(B, L, 16).cpu().numpy()
        hit = (ti == targets[:, :L, None]).any(axis=2)
        orc = np.where(hit, targets[:, :L], ti[:, :, 0])
        p1, p16 = w.recall_profile()
        accept.update({
            "top1_path": round(float(acceptance(ti[:, :, 0], targets).mean()), 3),
            "oracle_selector": round(float(acceptance(orc, targets).mean()), 3),
            "expected_top1": round(float(1 + np.cumprod(p1).sum()), 3),
            "expected_oracle_selector": round(float(1 + np.cumprod(p16).sum()), 3)})
    out = {
        "metric": "draft-select-verify blocks/s at B=64,L=8,V=151936; % MFMA / HBM roofline",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "L": L, "H": H, "V": V, "r": w.r,
                   "convs": w.n_convs, "conv_groups": w.groups if w.dynamic else 0, "topk": 16,
                   "gate": w.gate, "walk": w.walk, "temperature": w.temperature,
                   "launch": "hip-graph" if graphK is not None else "eager",
                   "pair_walk": "fused" if fused else "separate", "lm_head_w": w_layout,
                   "lm_head_out": form,
                   "rejection": ("two-pass" if two_pass else a.rejection) if sampled else None},
        "tokens_per_s": round(M / (ms_step * 1e-3), 1),
        "accepted_tokens_per_s": round(float(acc.sum()) / (ms_step * 1e-3), 1),
        "mean_accept_len": round(float(acc.mean()), 3),
        "accept_len": accept,
        "settle": {"steps": settle_steps, "seconds": round(settle_s, 2)},
        "gemm_ms": {"mean": round(float(np.mean(gemm_ms)), 4),
                    "min": round(float(np.min(gemm_ms)), 4),
                    "max": round(float(np.max(gemm_ms)), 4),
                    "source": "events around its launch in the stage pass after the timed region"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_pass_ms_per_step": round(stage_wall_ms, 4),
        "stage_pass_step_ms": {"p10": round(pct(0.1), 4), "median": round(pct(0.5), 4),
                               "p90": round(pct(0.9), 4)},
        "stage_hbm_gbs": hbm,
        "stage_roofline": stage_roof,
        "roofline": roof,
    }
    if w.dynamic and w.groups > 1:
        # the per-group corrections are a [M x H] x [H x 2G] product per application
        conv_flops = w.n_convs * 2.0 * M * H * 2 * w.groups
        out["stage_tflops"] = {"conv": round(conv_flops / (stage_ms["conv"] * 1e-3) / 1e12, 1)}
    out["cpu_baseline"] = cpu
    line = json.dumps(out)
    print(line, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
