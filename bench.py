#!/usr/bin/env python3
"""Benchmark of the DFlash 2 draft-select-verify step on one MI355X.

One step = one pass of the whole hot path over one batch:
  two-tap conv(s) -> LM-head logits -> top-16 -> [context gate] -> pair
  scores -> path walk (max-plus, or greedy with --walk greedy / the gated
  workload) -> greedy verification,
each stage a call into libdflash2 on the current HIP stream.  Scores, walk
and greedy verification run as one fused launch; a sampled walk runs scores
and walk as one launch, then a rejection verification that computes the
target rows' log-sum-exp itself, only for the rows its test reaches
(--separate: scores, walk and verification as separate launches, and for a
sampled walk an lse pass over every target row before the verification).  Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints ONE JSON line (rank 0, N = 1):
  value = blocks/s over the timed steps (B / seconds per step), the step
  captured once as a HIP graph and replayed (--eager: plain launches);
  a bf16 LM-head weight is packed once into the GEMM's tile layout before
  timing (--row-major-w: read as given);
  stage_ms = per-stage times from a second, eager pass with events;
  roofline = the LM-head GEMM kernel (the dominant kernel) against the bf16
  matrix-core peak (against HBM when its flop per algorithmic byte is below
  the ridge, as for the 4b-head workload), its duration measured with HIP
  events on its stream;
  cpu_baseline = the CPU oracle on a bounded block sample, same inputs.

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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_gemm_27b_head_traffic.txt")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=[0, 1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--walk", choices=["viterbi", "greedy"], default=None,
                    help="path walk (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-blocks", type=int, default=64,
                    help="blocks the CPU oracle runs for the baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--separate", action="store_true",
                    help="pair scores, walk and verification as separate launches, and for a "
                         "sampled walk the lse pass over every target row before the "
                         "verification (default: fused scores + walk, lazy verification)")
    ap.add_argument("--row-major-w", action="store_true",
                    help="LM-head GEMM reads W [V, H] as given (default for bf16: W packed once, "
                         "before timing, into the GEMM's 256 x 64 tile layout)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of the captured step")
    return ap.parse_args(argv)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "block_drafting_amd", "csrc", "lmhead.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str, w_layout: str):
    """HBM bytes per GEMM launch from the committed counter summary, if it
    was taken on this workload and W layout with the current kernel source;
    else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        m = re.match(r"^\s*([a-z0-9_]+)\s*[:=]\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if (kv.get("kernel_source_sha256_16") != kernel_source_hash() or kv.get("workload") != workload
            or kv.get("w_layout") != w_layout):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
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


def cpu_baseline(w, inp, n_blocks: int):
    """The CPU oracle (test infrastructure) on a bounded block sample."""
    import threadpoolctl
    import oracle as O
    import workloads as WL

    blocks = np.arange(min(n_blocks, w.B))
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] + [1])
    t0 = time.perf_counter()
    ora = O.run_step_front(w, inp, blocks)
    if w.temperature > 0:
        zt = WL.planted_target_logits(w, ora["top_idx"], blocks)
        O.rejection_verify(ora["path_tok"], ora["q"], ora["top_idx"], zt, w.temperature,
                           inp["u_acc"][blocks], inp["u_res"][blocks])
    else:
        tgt = WL.make_targets(w, ora["top_idx"], ora["path_tok"])
        O.verify_greedy(ora["path_tok"], tgt)
    dt = time.perf_counter() - t0
    return {"value": len(blocks) / dt, "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {len(blocks)} of {w.B} blocks of the {w.name} workload "
                      f"(full conv, logits over all {w.V} tokens, top-16, pairs, path, verify), "
                      f"{dt:.1f} s, fp64 numpy/OpenBLAS with {cores} threads"}


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
    buf = bd.StepBuffers(B, L, H, V, tdt, "cuda", n_convs=w.n_convs, keep_logits=True,
                         gate_rank=w.r if w.gate else 0, sample=sampled)
    tilemax = torch.empty((M, (V + bd.TILEMAX_COLS - 1) // bd.TILEMAX_COLS), dtype=torch.float32,
                          device="cuda")
    if sampled:
        u_path, u_acc, u_res = (dev(inp[k], "f32") for k in ("u_path", "u_acc", "u_res"))

    # one untimed step gives the candidates the verification targets are planted on
    bd.run_step(buf, x, convs, W, U, Vf, anchor, None, Wg=Wg, walk=w.walk,
                temperature=w.temperature, u_path=u_path if sampled else None)
    torch.cuda.synchronize()
    cand = buf.top_idx.view(B, L, 16).cpu().numpy()
    if sampled:
        # the target model's logits for every drafted position (+ the bonus one)
        z_target = torch.from_numpy(WL.planted_target_logits(w, cand)).cuda()
    else:
        target = torch.from_numpy(WL.make_targets(w, cand, buf.path_tok.cpu().numpy())).cuda()

    fused = not a.separate                 # scores + walk (+ greedy verification) in one launch
    two_pass = sampled and a.separate      # lse of every target row, then the verification
    if fused:
        tail = ["pair_sample", "verify"] if sampled else ["pair_select_verify"]
    else:
        tail = ["pair", "select"] + (["lse"] if two_pass else []) + ["verify"]
    order = ["conv", "gemm", "topk"] + (["gate"] if w.gate else []) + tail
    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)] for k in order}
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]

    def step(i=None):
        cur = x
        if i is not None:
            ev["conv"][i].record()
        for j, c in enumerate(convs):
            out = buf.y[j % len(buf.y)]
            if c["projT"] is not None:
                bd.twotap_conv_mm(cur, c["k0"], c["k1"], c["projT"], c["anchor_h"], out=out)
            else:
                bd.twotap_conv(cur, c["k0"], c["k1"], c["anchor_h"], c["proj"], c["groups"], out=out)
            cur = out
        if i is not None:
            ev["gemm"][i].record()
        bd.lmhead_logits_tilemax(cur.view(M, H), W, buf.logits, tilemax)
        if i is not None:
            ev["topk"][i].record()
        bd.topk16_tilemax(buf.logits, tilemax, buf.top_val, buf.top_idx)
        gate = None
        if w.gate:
            if i is not None:
                ev["gate"][i].record()
            gate = bd.context_gate(cur.view(M, H), Wg, buf.gate)
        ti = buf.top_idx.view(B, L, 16)
        if fused and sampled:
            # scores and the sampling walk in one launch, then the lazy verification
            if i is not None:
                ev["pair_sample"][i].record()
            bd.pair_sample(buf.top_val.view(B, L, 16), ti, anchor, U, Vf, u_path, w.temperature,
                           gate, None, None, buf.path_slot, buf.path_tok, buf.q)
            if i is not None:
                ev["verify"][i].record()
            bd.verify_rejection_lazy(buf.path_slot, buf.path_tok, buf.q, ti, z_target,
                                     w.temperature, u_acc, u_res, buf.accept_len, buf.next_tok)
            if i is not None:
                ev_end[i].record()
            return
        if fused:
            # scores, walk and verification in one launch; the scores stay on chip
            if i is not None:
                ev["pair_select_verify"][i].record()
            bd.pair_select_verify(buf.top_val.view(B, L, 16), ti, anchor, U, Vf, target, gate,
                                  w.walk, None, None, buf.path_slot, buf.path_tok,
                                  buf.path_score, buf.accept_len, buf.next_tok)
            if i is not None:
                ev_end[i].record()
            return
        if i is not None:
            ev["pair"][i].record()
        bd.pair_score(buf.top_val.view(B, L, 16), ti, anchor, U, Vf, buf.S0, buf.S, gate=gate)
        if i is not None:
            ev["select"][i].record()
        if sampled:
            bd.path_sample(buf.S0, buf.S, ti, u_path, w.temperature, buf.path_slot, buf.path_tok, buf.q)
            if i is not None:
                ev["lse"][i].record()
            bd.target_lse(z_target, w.temperature, buf.lse)
            if i is not None:
                ev["verify"][i].record()
            bd.verify_rejection(buf.path_slot, buf.path_tok, buf.q, ti, z_target, buf.lse,
                                w.temperature, u_acc, u_res, buf.accept_len, buf.next_tok)
        else:
            bd.path_select(buf.S0, buf.S, ti, buf.path_slot, buf.path_tok, buf.path_score, mode=w.walk)
            if i is not None:
                ev["verify"][i].record()
            bd.verify_greedy(buf.path_tok, target, buf.accept_len, buf.next_tok)
        if i is not None:
            ev_end[i].record()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    outs = (buf.top_val, buf.top_idx, buf.path_slot, buf.path_tok, buf.accept_len, buf.next_tok)
    eager_out = [t.clone() for t in outs]

    # The whole step captured once as a HIP graph (every call enqueues on the
    # current stream, nothing allocates or clears memory), then replayed:
    # the timed loop pays no per-kernel launch cost on the host.
    graph = None
    if not a.eager:
        try:
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                step()
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=cap):
                    step()
            torch.cuda.current_stream().wait_stream(cap)
            torch.cuda.synchronize()
            for _ in range(a.warmup):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # pragma: no cover - capture unsupported
            log(f"[bench] graph capture failed ({e}); timing eager steps")
            graph = None
    run = graph.replay if graph is not None else step
    log(f"[bench] warmup done ({a.warmup} steps); timing {a.steps} steps "
        f"({'graph replays' if graph is not None else 'eager'})")
    t_start = time.perf_counter()
    for _ in range(a.steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] timed {a.steps} steps in {wall:.3f} s")
    for t, r in zip(outs, eager_out):          # the replays computed what eager steps do
        assert torch.equal(t, r), "graph replay differs from the eager step"

    # light sanity on the last step's outputs
    acc = buf.accept_len.cpu().numpy()
    tv = buf.top_val.cpu().numpy()
    assert ((acc >= 1) & (acc <= L + 1)).all() and (np.diff(tv, axis=1) <= 0).all()

    # per-stage times: a second pass of eager steps with events between stages
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    stage_ms = {k: 0.0 for k in order}
    for i in range(a.steps):
        marks = [ev[k][i] for k in order] + [ev_end[i]]
        for k, s, e in zip(order, marks[:-1], marks[1:]):
            stage_ms[k] += s.elapsed_time(e) / a.steps
    ms_step = wall * 1e3 / a.steps
    gemm_s = stage_ms["gemm"] * 1e-3
    flops = 2.0 * M * H * V
    # algorithmic GEMM bytes: W and h read once, logits and tile maxima written
    gemm_bytes = (V * H + M * H) * (2 if bf16 else 4) + M * V * 4 + M * ((V + 255) // 256) * 4
    if bf16 and flops / gemm_bytes < PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        # below the ridge (small M): HBM-bound
        achieved = gemm_bytes / gemm_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(w.name, w_layout)}
    elif bf16:
        achieved = flops / gemm_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(w.name, w_layout)}
    else:
        achieved = flops / gemm_s / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_F32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F32_TFLOPS, 5), "traffic": None}
    # algorithmic HBM rates of the streaming stages
    es = 2 if bf16 else 4
    conv_bytes = w.n_convs * (2 * L + 1) * B * H * es
    if w.dynamic and w.groups > 1:
        conv_bytes += w.n_convs * 2 * w.groups * H * es      # the correction maps
    # (the top-16 reads only the tiles its maxima allow, ~1/37 of the logits
    # at V = 151936, so no HBM rate is quoted for it)
    hbm = {"conv": round(conv_bytes / (stage_ms["conv"] * 1e-3) / 1e9, 1)}
    if two_pass:
        hbm["lse"] = round(B * (L + 1) * V * 4 / (stage_ms["lse"] * 1e-3) / 1e9, 1)
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
                   "launch": "hip-graph" if graph is not None else "eager",
                   "pair_walk": "fused" if fused else "separate", "lm_head_w": w_layout,
                   "rejection": ("two-pass" if two_pass else "lazy") if sampled else None},
        "tokens_per_s": round(M / (ms_step * 1e-3), 1),
        "accepted_tokens_per_s": round(float(acc.sum()) / (ms_step * 1e-3), 1),
        "mean_accept_len": round(float(acc.mean()), 3),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_hbm_gbs": hbm,
        "roofline": roof,
    }
    if w.dynamic and w.groups > 1:
        # the per-group corrections are a [M x H] x [H x 2G] product per application
        conv_flops = w.n_convs * 2.0 * M * H * 2 * w.groups
        out["stage_tflops"] = {"conv": round(conv_flops / (stage_ms["conv"] * 1e-3) / 1e12, 1)}
    if not a.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {a.cpu_blocks} blocks")
        out["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_blocks)
    else:
        out["cpu_baseline"] = None
    line = json.dumps(out)
    print(line, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
