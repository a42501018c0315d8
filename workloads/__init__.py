"""Seeded synthetic workloads for the DFlash 2 draft-select-verify step.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no convolution, logits, top-k, scoring, path walk or
verification).  Both the CPU oracle and the HIP path read the same arrays
from here, so they see bit-identical inputs.

Representation
--------------
* fp32 tensors are ``numpy.float32`` arrays.
* bf16 tensors are ``numpy.uint16`` arrays holding the raw bf16 bit patterns
  (rounded from fp32 by round-to-nearest-even).  Each consumer decodes them
  itself.
* token ids are ``numpy.int32``.

Random streams
--------------
Every tensor has its own PCG64 stream keyed by ``(seed, tensor_tag)``; large
tensors are filled in a fixed number of chunks, each with its own child key,
so the values do not depend on how many threads fill them.

The workloads
-------------
0. tiny: 1 block, L=8, H=256, V=4096, r=32, fp32 end to end.
1. 4B-shaped head: 32 blocks, L=8, H=2560, V=151936, r=64, bf16.
2. 27B-shaped head: 64 blocks, L=8, H=5120, V=151936, r=64, bf16.
3. conv-heavy body: 128 blocks, L=16, H=5120, 20 chained dynamic convs, r=64.
4. stress: 256 blocks, L=16, H=5120, r=128, logits on a 1/64 grid (ties),
   targets a 50/50 mix of all-correct and random-miss blocks.
5. 27B-shaped head with the pages' own selector: rank-256 factors weighted
   by a context gate from the final hidden state, greedy best-successor walk.
6. conv-heavy body with one correction pair per 16 channels (G = H/16), the
   correction map stored transposed in bf16.
7. 27B-shaped head sampled at T = 1, verified losslessly against synthetic
   target logits (planted tokens over noise).

The planted-target recall profile of workloads 0-2 and 4 is the per-position
Recall@1 / Recall@16 of Table 1 of "DFlash 2: Keep Drafting Parallel"
(section "The right token is already in the candidates"), extended to L=8 by
holding the last value.  "N(0, s)" in the workload descriptions is read with
s as the variance.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import numpy as np

BASE_SEED = 20260818
_CHUNKS = 64  # fixed fill granularity: values never depend on thread count

# Per-position Recall@1 and Recall@16 of the pages' Table 1 (positions 0-6).
TABLE1_RECALL1 = (0.854, 0.803, 0.794, 0.783, 0.775, 0.759, 0.729)
TABLE1_RECALL16 = (0.995, 0.973, 0.948, 0.926, 0.908, 0.894, 0.878)
# The rounded profile the workloads use (positions 0-6), held at L=8.
PROFILE_P1 = (0.85, 0.80, 0.79, 0.78, 0.77, 0.76, 0.73)
PROFILE_P16 = (0.995, 0.97, 0.95, 0.93, 0.91, 0.89, 0.88)


def hold_last(profile: Sequence[float], L: int) -> np.ndarray:
    """Extend a per-position profile to L positions by repeating its last value."""
    p = list(profile)[:L]
    while len(p) < L:
        p.append(profile[-1])
    return np.asarray(p, dtype=np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    B: int
    L: int
    H: int
    V: int
    r: int
    dtype: str            # "f32" or "bf16"
    n_convs: int          # chained conv applications
    dynamic: bool         # conv taps corrected from x_t through a [H, 2] map
    target_mode: str      # "planted" or "mix"
    dyadic: bool          # integer / dyadic construction (exact sums, ties)
    parity_blocks: int    # seeded block subset the oracle checks at full size
    gate: bool = False    # pair match weighted by a context gate from h_t (Wg [r, H])
    walk: str = "viterbi"  # "viterbi" (max-plus), "greedy" (best successor), "sample"
    #                        (each position from its predecessor's row) or "sample-path"
    #                        (the whole path from exp(score / T))
    groups: int = 1       # correction groups of a dynamic conv (H/16: one per 16 channels)
    profile: str = "table1"  # recall profile: "table1" or "decay" (linear 0.85 -> 0.60)
    temperature: float = 0.0  # > 0: sampled walk and lossless rejection verification

    @property
    def M(self) -> int:
        return self.B * self.L

    @property
    def seed(self) -> int:
        return BASE_SEED + self.cid

    def recall_profile(self):
        """(p1, p16): per-position probabilities that the planted target is
        the top-1 candidate, and that it is inside the top-16."""
        if self.profile == "decay":
            p1 = 0.85 - 0.25 * np.arange(self.L) / (self.L - 1)
            p16 = np.maximum(hold_last(PROFILE_P16, self.L), p1)
            return p1, p16
        return hold_last(PROFILE_P1, self.L), hold_last(PROFILE_P16, self.L)

    def with_blocks(self, B: int) -> "Workload":
        """Same workload at another batch size (used for scaled sweeps and
        small CPU cases)."""
        return dataclasses.replace(self, B=B)

    def shrink(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[int, Workload] = {
    0: Workload(0, "tiny", 1, 8, 256, 4096, 32, "f32", 1, False, "planted", False, 1),
    1: Workload(1, "4b-head", 32, 8, 2560, 151936, 64, "bf16", 1, False, "planted", False, 32),
    2: Workload(2, "27b-head", 64, 8, 5120, 151936, 64, "bf16", 1, False, "planted", False, 8),
    3: Workload(3, "conv-heavy", 128, 16, 5120, 151936, 64, "bf16", 20, True, "planted", False, 4,
                profile="decay"),
    4: Workload(4, "stress", 256, 16, 5120, 151936, 128, "bf16", 1, False, "mix", True, 4),
    # The pages' own selector on the 27B-shaped head: rank-256 factors, the
    # context gate and the greedy best-successor walk.
    5: Workload(5, "27b-gated-greedy", 64, 8, 5120, 151936, 256, "bf16", 1, False, "planted",
                False, 8, gate=True, walk="greedy"),
    # The conv-heavy body with the post's own coefficients: one correction
    # pair per 16 channels (320 groups at H = 5120).
    6: Workload(6, "conv-heavy-g16", 128, 16, 5120, 151936, 64, "bf16", 20, True, "planted",
                False, 4, groups=320, profile="decay"),
    # Sampling at T = 1 (the post's Table 2 T = 1 column) with lossless
    # rejection verification against synthetic target logits.
    7: Workload(7, "27b-sampled", 64, 8, 5120, 151936, 64, "bf16", 1, False, "logits", False, 8,
                walk="sample", temperature=1.0),
    # The same with the whole path drawn from exp(score / T) over all 16^L
    # paths (the sampling twin of the max-plus walk).
    8: Workload(8, "27b-sampled-path", 64, 8, 5120, 151936, 64, "bf16", 1, False, "logits", False,
                8, walk="sample-path", temperature=1.0),
}


# ---------------------------------------------------------------- streams
def _rng(seed: int, tag: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, chunk])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_chunked(n: int, seed: int, tag: int, fn) -> np.ndarray:
    """Fill a float32 array of n values chunk by chunk; chunk c uses stream
    (seed, tag, c) and fn(gen, out_view) to fill its slice."""
    out = np.empty(n, dtype=np.float32)
    if n < (1 << 20):
        fn(_rng(seed, tag, 0), out)
        return out
    bounds = np.linspace(0, n, _CHUNKS + 1).astype(np.int64)

    def work(c):
        fn(_rng(seed, tag, c), out[bounds[c]:bounds[c + 1]])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(_CHUNKS)))
    return out


def normal_f32(shape, var: float, seed: int, tag: int) -> np.ndarray:
    n = int(np.prod(shape))
    std = np.float32(np.sqrt(var))

    def fn(g, out):
        g.standard_normal(out=out, dtype=np.float32)
        out *= std

    return _fill_chunked(n, seed, tag, fn).reshape(shape)


def rounded_normal_f32(shape, var: float, clip: float, seed: int, tag: int) -> np.ndarray:
    """round(N(0, var)) clipped to [-clip, clip]: small integers as float32."""
    a = normal_f32(shape, var, seed, tag)
    np.rint(a, out=a)
    np.clip(a, -clip, clip, out=a)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (via torch's cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# Tensor tags (stable: changing them changes every workload).
TAG_X, TAG_ANCHOR_H, TAG_K0, TAG_K1, TAG_PROJ, TAG_W, TAG_U, TAG_V = range(1, 9)
TAG_ANCHOR_TOK, TAG_TARGET, TAG_WG, TAG_UNIFORM, TAG_ZTARGET = 9, 10, 11, 12, 13
TAG_CONV_STRIDE = 16  # conv j of a chain uses tags TAG_* + TAG_CONV_STRIDE * j


def make_inputs(w: Workload, with_head: bool = True) -> Dict[str, object]:
    """All inputs of one step except the verification targets.

    Returns a dict with
      x        [B, L, H]   activations entering the first conv
      convs    list of n_convs dicts {anchor_h [B,H], k0 [H], k1 [H], proj [H,2] or None,
               groups, projT}: with groups > 1 the correction map is given as
               projT [2*groups, H] in the storage dtype (proj is None)
      W        [V, H]      LM-head weight (omitted when with_head is False)
      U, Vf    [V, r]      low-rank pair factors (omitted when with_head is False)
      Wg       [r, H]      context-gate map, N(0, 1/H) (gated workloads only)
      anchor_tok [B]       last verified token id of each block
      u_path, u_acc [B, L], u_res [B]   uniforms (sampled workloads only)
    Activation and weight tensors are bf16 bits or fp32 according to w.dtype.
    """
    B, L, H, V, r, s = w.B, w.L, w.H, w.V, w.r, w.seed
    bf16 = w.dtype == "bf16"

    def act(shape, tag):
        if w.dyadic:
            a = rounded_normal_f32(shape, 1.0, 4.0, s, tag)
        else:
            a = normal_f32(shape, 1.0, s, tag)
        return to_bf16_bits(a) if bf16 else a

    out: Dict[str, object] = {"x": act((B, L, H), TAG_X)}
    convs = []
    for j in range(w.n_convs):
        o = TAG_CONV_STRIDE * j
        if w.dyadic:
            k0 = rounded_normal_f32((H,), 0.5, 2.0, s, TAG_K0 + o)
            k1 = rounded_normal_f32((H,), 0.5, 2.0, s, TAG_K1 + o)
        else:
            k0 = normal_f32((H,), 0.5, s, TAG_K0 + o)
            k1 = normal_f32((H,), 0.5, s, TAG_K1 + o)
        proj = projT = None
        if w.dynamic and w.groups == 1:
            proj = normal_f32((H, 2), 0.01 / H, s, TAG_PROJ + o)
        elif w.dynamic:
            projT = normal_f32((2 * w.groups, H), 0.01 / H, s, TAG_PROJ + o)
            projT = to_bf16_bits(projT) if bf16 else projT
        convs.append({"anchor_h": act((B, H), TAG_ANCHOR_H + o), "k0": k0, "k1": k1,
                      "proj": proj, "projT": projT, "groups": w.groups})
    out["convs"] = convs
    if with_head:
        if w.dyadic:
            # W = b/64, U = c/8, V = d/8 with small integers b, c, d.
            Wv = rounded_normal_f32((V, H), 1.0, 8.0, s, TAG_W) / np.float32(64.0)
            Uv = rounded_normal_f32((V, w.r), 6.4, 8.0, s, TAG_U) / np.float32(8.0)
            Vv = rounded_normal_f32((V, w.r), 6.4, 8.0, s, TAG_V) / np.float32(8.0)
        else:
            Wv = normal_f32((V, H), 1.0 / H, s, TAG_W)
            Uv = normal_f32((V, r), 0.1, s, TAG_U)
            Vv = normal_f32((V, r), 0.1, s, TAG_V)
        if bf16:
            Wv, Uv, Vv = to_bf16_bits(Wv), to_bf16_bits(Uv), to_bf16_bits(Vv)
        out["W"], out["U"], out["Vf"] = Wv, Uv, Vv
        if w.gate:
            Wg = normal_f32((r, H), 1.0 / H, s, TAG_WG)
            out["Wg"] = to_bf16_bits(Wg) if bf16 else Wg
    out["anchor_tok"] = _rng(s, TAG_ANCHOR_TOK).integers(0, V, size=B, dtype=np.int32)
    if w.temperature > 0:
        out.update(make_uniforms(w))
    return out


def parity_subset(w: Workload) -> np.ndarray:
    """Seeded, sorted subset of block indices the oracle checks at full size."""
    g = _rng(w.seed, 99)
    k = min(w.parity_blocks, w.B)
    return np.sort(g.permutation(w.B)[:k]).astype(np.int64)


def select_blocks(inp: Dict[str, object], blocks: np.ndarray) -> Dict[str, object]:
    """The inputs restricted to a subset of blocks (weights shared)."""
    out = dict(inp)
    out["x"] = inp["x"][blocks]
    out["convs"] = [dict(c, anchor_h=c["anchor_h"][blocks]) for c in inp["convs"]]
    out["anchor_tok"] = inp["anchor_tok"][blocks]
    for k in ("u_path", "u_acc", "u_res"):
        if k in inp:
            out[k] = inp[k][blocks]
    return out


# ---------------------------------------------------------------- targets
def planted_targets(top_idx: np.ndarray, V: int, p1: np.ndarray, p16: np.ndarray,
                    seed: int, tag: int = TAG_TARGET) -> np.ndarray:
    """Planted verifier argmax per position, given each position's 16
    candidates top_idx [B, L, 16] (slot 0 = top-1).

    Per block and position, independently: with probability p1[t] the target
    is candidate slot 0; with probability p16[t] - p1[t] it is a uniform slot
    in 1..15; otherwise it is a uniform token outside the 16 candidates.  The
    bonus token target[:, L] is uniform over the vocabulary.
    Returns int32 [B, L + 1].
    """
    B, L, K = top_idx.shape
    g = _rng(seed, tag)
    u = g.random((B, L))
    slot = g.integers(1, K, size=(B, L))
    rand_tok = g.integers(0, V, size=(B, L))
    bonus = g.integers(0, V, size=B)
    tgt = np.empty((B, L + 1), dtype=np.int32)
    for b in range(B):
        for t in range(L):
            cands = top_idx[b, t]
            if u[b, t] < p1[t]:
                tgt[b, t] = cands[0]
            elif u[b, t] < p16[t]:
                tgt[b, t] = cands[slot[b, t]]
            else:
                tok = int(rand_tok[b, t])
                while tok in cands:          # resample outside the candidates
                    tok = int(g.integers(0, V))
                tgt[b, t] = tok
        tgt[b, L] = bonus[b]
    return tgt


def mixed_targets(path_tok: np.ndarray, V: int, seed: int, tag: int = TAG_TARGET) -> np.ndarray:
    """50/50 per block: all-correct (target = path for t < L) or random-miss
    (target = path before a uniform miss position m, a different token at m,
    uniform tokens after).  The bonus token is uniform.  Returns [B, L + 1]."""
    B, L = path_tok.shape
    g = _rng(seed, tag)
    allc = g.random(B) < 0.5
    miss = g.integers(0, L, size=B)
    rest = g.integers(0, V, size=(B, L + 1))
    tgt = rest.astype(np.int32)
    for b in range(B):
        m = L if allc[b] else int(miss[b])
        tgt[b, :m] = path_tok[b, :m]
        if m < L:
            tok = int(rest[b, m])
            while tok == path_tok[b, m]:
                tok = int(g.integers(0, V))
            tgt[b, m] = tok
    return tgt


def make_uniforms(w: Workload) -> Dict[str, np.ndarray]:
    """The sampled walk's and the rejection step's random numbers, drawn here
    and passed to both sides: u_path [B, L], u_acc [B, L], u_res [B], float32
    in [0, 1)."""
    g = _rng(w.seed, TAG_UNIFORM)
    top = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))

    def unif(shape):
        return np.minimum(g.random(shape).astype(np.float32), top)

    return {"u_path": unif((w.B, w.L)), "u_acc": unif((w.B, w.L)), "u_res": unif((w.B,))}


# Target logits: N(0, 1) noise plus a bump on the planted token.  With V =
# 151936 the bump of 15 gives the planted token about 93% of the target's
# probability at T = 1.
TARGET_BUMP = 15.0


def planted_target_logits(w: Workload, top_idx: np.ndarray, blocks: Optional[np.ndarray] = None
                          ) -> np.ndarray:
    """Synthetic target logits [Bs, L + 1, V] (float32) for the given blocks'
    candidates top_idx [Bs, L, 16]: the planted token of each position is
    chosen as planted_targets chooses it (same recall profile, same streams)
    and gets TARGET_BUMP over N(0, 1) noise drawn per block."""
    Bs, L, _ = top_idx.shape
    blocks = np.arange(Bs) if blocks is None else np.asarray(blocks)
    p1, p16 = w.recall_profile()
    planted = planted_targets(top_idx, w.V, p1, p16, w.seed)     # [Bs, L + 1]
    z = np.empty((Bs, L + 1, w.V), dtype=np.float32)
    for i, b in enumerate(blocks):
        z[i] = normal_f32((L + 1, w.V), 1.0, w.seed, TAG_ZTARGET * 1000003 + int(b))
        z[i, np.arange(L + 1), planted[i]] += np.float32(TARGET_BUMP)
    return z


def make_targets(w: Workload, top_idx: np.ndarray, path_tok: Optional[np.ndarray]) -> np.ndarray:
    """Targets of workload w: planted from the candidates, or the 50/50 mix
    built around a path (workload 4)."""
    if w.target_mode == "mix":
        assert path_tok is not None
        return mixed_targets(path_tok, w.V, w.seed)
    p1, p16 = w.recall_profile()
    return planted_targets(top_idx, w.V, p1, p16, w.seed)
