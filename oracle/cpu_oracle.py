"""Plain CPU oracle of the DFlash 2 draft-select-verify step (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the HIP product path shares no code with it.

Sources (cited by page title and section):
  [POST]   "DFlash 2: Keep Drafting Parallel" (Inco AI; Chinese translations
           on the mynewscn and twiscan pages).
  [GLONCE] "Inco AI's DFlash 2 lifts LLM decoding output 16-25%" (Glonce).

Readings of points the pages leave open are stated where they are used.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

K = 16  # candidates kept per position ([POST] "A lightweight path selector")


# ------------------------------------------------------------------ numbers
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64: a bf16 number is the
    upper half of an IEEE single."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even; result in fp64.

    bf16 keeps 8 significant bits, so a value in [2^(e-1), 2^e) is rounded to
    a multiple of 2^(e-8); below the smallest normal (2^-126) the spacing stays
    2^-133.  Values past the largest finite bf16 after rounding become inf.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.maximum(e, -125)
    q = np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)
    big = np.abs(q) > _BF16_MAX
    if np.any(big):
        q = np.where(big, np.copysign(np.inf, q), q)
    return q


def round_to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values once to the storage type ("bf16" or "f32"); fp64 out."""
    if dtype == "bf16":
        return round_to_bf16(v)
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def as_f64(a, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored tensor (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------------------ a1 conv
def twotap_conv(x: np.ndarray, anchor_h: Optional[np.ndarray], k0: np.ndarray,
                k1: np.ndarray, proj: Optional[np.ndarray] = None,
                groups: int = 1) -> np.ndarray:
    """Two-tap dynamic depthwise convolution over one block, exact in fp64.

    [POST] "A lightweight local convolution", eq. Conv_k: every position t
    mixes its own representation with its predecessor's through two
    per-channel taps,  y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}.
    Each tap is a learnable base tap plus a small correction computed from the
    current hidden state x_t, one correction shared by a group of channels
    (the post shares one per 16 channels; the conv-heavy workload uses a single
    [H x 2] projection, i.e. one group).  Position 0 reads the last verified
    token's representation (the anchor) in place of x_{-1} (same section and
    Fig. 4).

    Readings: the correction is linear in x_t with no bias or activation
    (Delta[t, g, j] = sum_c x_t[c] * proj[c, 2g + j]); channel c belongs to
    group c // (H / groups); no residual is added; a missing anchor is zero
    and a missing proj means static taps.

    x [B, L, H], anchor_h [B, H] or None, k0/k1 [H], proj [H, 2*groups] or
    None, all fp64.  Returns the exact y [B, L, H] in fp64 (unrounded).
    """
    B, L, H = x.shape
    if anchor_h is None:
        anchor_h = np.zeros((B, H))
    prev = np.concatenate([anchor_h[:, None, :], x[:, :-1, :]], axis=1)
    if proj is None:
        c0 = np.broadcast_to(k0, (B, L, H))
        c1 = np.broadcast_to(k1, (B, L, H))
    else:
        delta = (x.reshape(B * L, H) @ proj).reshape(B, L, groups, 2)
        group_of_channel = np.arange(H) // (H // groups)
        c0 = k0[None, None, :] + delta[:, :, group_of_channel, 0]
        c1 = k1[None, None, :] + delta[:, :, group_of_channel, 1]
    return c0 * x + c1 * prev


def conv_chain(x: np.ndarray, convs, dtype: str) -> np.ndarray:
    """Chained conv applications as the drafter body places them, one before
    and one after each sublayer ([POST] "A lightweight local convolution",
    Fig. 4); the sublayers themselves need trained weights and are taken as
    identity.  Each application's output is rounded once to the storage type
    and feeds the next.  x fp64 [B, L, H]; returns fp64 values of the stored
    output."""
    y = x
    for c in convs:
        ah = c["anchor_h"]
        y = round_to_dtype(twotap_conv(y, ah, c["k0"], c["k1"], c.get("proj"),
                                       c.get("groups", 1)), dtype)
    return y


# ------------------------------------------------------------------ a2 logits
def lm_logits(y: np.ndarray, W: np.ndarray, w_dtype: str, chunk_elems: int = 1 << 26) -> np.ndarray:
    """Drafter logits U_t(b) for every token b ([POST] "A lightweight path
    selector": the unary term is the drafter's own logit).

    z[m, n] = sum_c y[m, c] * W[n, c], evaluated in fp64 from the exact
    operand values and rounded once to fp32.  y [M, H] fp64; W [V, H] stored
    (bf16 bits or fp32), decoded a slice of rows at a time.  Returns fp32 [M, V].
    """
    M, H = y.shape
    V = W.shape[0]
    z = np.empty((M, V), dtype=np.float32)
    step = max(1, chunk_elems // H)
    for n0 in range(0, V, step):
        Wc = as_f64(W[n0:n0 + step], w_dtype)
        z[:, n0:n0 + step] = (y @ Wc.T).astype(np.float32)
    return z


# ------------------------------------------------------------------ a3 top-16
def canonical_logits(z: np.ndarray) -> np.ndarray:
    """Order-canonical copy of fp32 logits: -0 becomes +0 and NaN becomes
    -inf (reading: NaN ranks below every number)."""
    z = np.asarray(z, dtype=np.float32)
    z = np.where(np.isnan(z), np.float32(-np.inf), z)
    return z + np.float32(0.0)


def topk16(z: np.ndarray):
    """Top-16 candidates per row ([POST] "A lightweight path selector": the
    drafter keeps its 16 best tokens at every position).

    The first 16 indices of the row sorted by (value descending, index
    ascending): equal values go to the lowest token id first (the stress
    workload's tie rule).  Decided on the fp32 logits.  z [M, V] fp32.
    Returns (top_val fp32 [M, 16], top_idx int32 [M, 16]).
    """
    zc = canonical_logits(z)
    M, V = zc.shape
    idx = np.broadcast_to(np.arange(V), (M, V))
    order = np.lexsort((idx, -zc), axis=-1)[:, :K]
    return np.take_along_axis(zc, order, axis=1), order.astype(np.int32)


def topk_gaps(z: np.ndarray, top_val: np.ndarray) -> np.ndarray:
    """Per slot s, the smaller gap to its neighbours in the sorted order
    (slot 15 also against the 17th largest value): how far a candidate is
    from swapping with the next one.  Returns fp64 [M, 16]."""
    zc = canonical_logits(z).astype(np.float64)
    M = zc.shape[0]
    v17 = -np.sort(-zc, axis=1)[:, K]  # the 17th value
    vals = np.concatenate([top_val.astype(np.float64), v17[:, None]], axis=1)
    d = vals[:, :-1] - vals[:, 1:]              # gap below slot s
    up = np.concatenate([np.full((M, 1), np.inf), d[:, :-1]], axis=1)
    return np.minimum(up, d)


# ------------------------------------------------------------------ a4 pair scores
def pair_scores(top_val: np.ndarray, top_idx: np.ndarray, anchor_tok: Optional[np.ndarray],
                U: np.ndarray, Vf: np.ndarray, uv_dtype: str, gate: Optional[np.ndarray] = None):
    """Scores of every adjacent candidate pair ([POST] "A lightweight path
    selector", eq. S_t(a, b)): the candidate's own logit plus a low-rank
    match between the previous token a and the candidate b.

    In the workloads' ungated form the match is u_a . v_b with per-token
    factor tables U, V [vocab, r] (the post's context gate is taken as all
    ones).  Position 0's previous token is the last verified token (the walk
    starts from it); with anchor_tok None its match term is 0.

      S0[b, j]        = top_val[b, 0, j] + U[anchor_tok[b]] . V[top_idx[b, 0, j]]
      S[b, t-1, i, j] = top_val[b, t, j] + U[top_idx[b, t-1, i]] . V[top_idx[b, t, j]]

    With a context gate (the post's H(h_t), [B, L, r] values for the
    position of the current candidate), the match becomes
    sum_k U[a, k] * gate[b, t, k] * V[b', k]: A(a) (.) H(h_t) matched with B(b').

    Evaluated in fp64 from the exact inputs, rounded once to fp32.
    top_val fp32 [B, L, 16], top_idx int [B, L, 16].
    Returns S0 fp32 [B, 16], S fp32 [B, L-1, 16, 16].
    """
    Uf = as_f64(U, uv_dtype)
    Vff = as_f64(Vf, uv_dtype)
    tv = top_val.astype(np.float64)
    cu = Uf[top_idx]        # [B, L, 16, r]  factor of each candidate as "previous"
    cv = Vff[top_idx]       # [B, L, 16, r]  factor of each candidate as "current"
    g = None if gate is None else np.asarray(gate, dtype=np.float32).astype(np.float64)
    if anchor_tok is None:
        s0 = tv[:, 0, :]
    else:
        ua = Uf[np.asarray(anchor_tok)]                      # [B, r]
        if g is not None:
            ua = ua * g[:, 0, :]
        s0 = tv[:, 0, :] + np.einsum("br,bjr->bj", ua, cv[:, 0])
    prev = cu[:, :-1]
    if g is not None:
        prev = prev * g[:, 1:, None, :]                      # gate of position t
    match = np.einsum("btir,btjr->btij", prev, cv[:, 1:])
    S = tv[:, 1:, None, :] + match
    return s0.astype(np.float32), S.astype(np.float32)


def context_gate(y: np.ndarray, Wg: np.ndarray, w_dtype: str) -> np.ndarray:
    """Context gate H(h_t) of the gated pair score ([POST] "A lightweight
    path selector", eq. S_t(a, b): the gate, a function of the drafter's
    hidden state at position t, decides which channels of the match count).

    Reading: the pages give no form for H; the plainest gate is a logistic
    sigmoid of a linear map of h_t,
      gate[m, k] = 1 / (1 + exp(-sum_c y[m, c] * Wg[k, c])),
    evaluated in fp64 from the exact inputs and rounded once to fp32.
    y fp64 [M, H] (the hidden states the LM head reads), Wg [r, H] stored.
    Returns fp32 [M, r].
    """
    a = np.asarray(y, dtype=np.float64) @ as_f64(Wg, w_dtype).T
    return (1.0 / (1.0 + np.exp(-a))).astype(np.float32)


# ------------------------------------------------------------------ a5 path walk
def path_select(S0: np.ndarray, S: np.ndarray, top_idx: np.ndarray):
    """Exact max-plus (Viterbi) walk over the precomputed pair scores.

    [POST] "A lightweight path selector": the only serial step walks the
    precomputed scores from the last verified token to one path.  The post's
    walk follows the best successor greedily; the step built here takes the
    exact maximum over all 16^L slot paths of S0[p0] + sum_t S[t-1, p_{t-1}, p_t],
    by the max-plus recursion

      delta_0 = S0,  delta_t[j] = max_i fl32(delta_{t-1}[i] + S[t-1, i, j]),

    deciding in fp32 (the kernel's precision).  Ties go to the lowest slot at
    every maximum and at the final argmax, which selects, among optimal paths,
    the one smallest in (p_{L-1}, p_{L-2}, ..., p_0) order.

    S0 fp32 [B, 16], S fp32 [B, L-1, 16, 16], top_idx [B, L, 16].
    Returns (path_slot int32 [B, L], path_tok int32 [B, L], path_score fp32 [B]).
    """
    S0 = np.asarray(S0, dtype=np.float32)
    S = np.asarray(S, dtype=np.float32)
    B = S0.shape[0]
    L = S.shape[1] + 1
    delta = S0.copy()
    back = np.zeros((B, L, K), dtype=np.int64)
    for t in range(1, L):
        cand = delta[:, :, None] + S[:, t - 1]          # [B, i, j], fp32 sums
        back[:, t] = np.argmax(cand, axis=1)             # first (lowest) i at the max
        delta = np.take_along_axis(cand, back[:, t][:, None, :], axis=1)[:, 0]
    slot = np.zeros((B, L), dtype=np.int64)
    slot[:, L - 1] = np.argmax(delta, axis=1)
    score = delta[np.arange(B), slot[:, L - 1]]
    for t in range(L - 1, 0, -1):
        slot[:, t - 1] = back[np.arange(B), t, slot[:, t]]
    tok = np.take_along_axis(np.asarray(top_idx), slot[:, :, None], axis=2)[:, :, 0]
    return slot.astype(np.int32), tok.astype(np.int32), score.astype(np.float32)


def path_select_greedy(S0: np.ndarray, S: np.ndarray, top_idx: np.ndarray):
    """The post's own walk ([POST] "A lightweight path selector"; [GLONCE]
    names a greedy choice as one way the serial walk ends): start from the last
    verified token and at every position take the best successor of the
    token chosen before,

      p_0 = argmax_j S0[j],  p_t = argmax_j S[t-1, p_{t-1}, j],

    lowest slot on ties.  The returned score is the fp32 running sum
    S0[p_0] + S[0, p_0, p_1] + ... in position order.
    Returns (path_slot int32 [B, L], path_tok int32 [B, L], path_score fp32 [B]).
    """
    S0 = np.asarray(S0, dtype=np.float32)
    S = np.asarray(S, dtype=np.float32)
    B = S0.shape[0]
    L = S.shape[1] + 1
    b = np.arange(B)
    slot = np.zeros((B, L), dtype=np.int64)
    slot[:, 0] = np.argmax(S0, axis=1)
    score = S0[b, slot[:, 0]].copy()
    for t in range(1, L):
        row = S[b, t - 1, slot[:, t - 1]]                  # [B, 16] successors of p_{t-1}
        slot[:, t] = np.argmax(row, axis=1)
        score = (score + row[b, slot[:, t]]).astype(np.float32)
    tok = np.take_along_axis(np.asarray(top_idx), slot[:, :, None], axis=2)[:, :, 0]
    return slot.astype(np.int32), tok.astype(np.int32), score.astype(np.float32)


def greedy_margin(S0: np.ndarray, S: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """Smallest gap, along a greedy walk's slots, between the chosen entry and
    the runner-up of the row it was chosen from (fp64, [B]).  A perturbation
    of the scores smaller than half of it cannot change the walk."""
    S0 = np.asarray(S0, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    B, L = slot.shape
    b = np.arange(B)

    def gap(row):
        srt = -np.sort(-row, axis=1)
        return srt[:, 0] - srt[:, 1]

    m = gap(S0)
    for t in range(1, L):
        m = np.minimum(m, gap(S[b, t - 1, slot[:, t - 1]]))
    return m


def path_scores_f64(S0: np.ndarray, S: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """fp64 score of given slot paths: S0[p0] + sum_t S[t-1, p_{t-1}, p_t]."""
    S0 = np.asarray(S0, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    B, L = slot.shape
    b = np.arange(B)
    sc = S0[b, slot[:, 0]]
    for t in range(1, L):
        sc = sc + S[b, t - 1, slot[:, t - 1], slot[:, t]]
    return sc


def path_margin(S0: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Gap between the best and the second-best path score, in fp64.

    Forward maxima alpha_t[j] (best score of a prefix ending at slot j) and
    backward maxima beta_t[j] (best score of a suffix leaving slot j) give
    mu_t[j] = alpha_t[j] + beta_t[j], the best score of any path through j
    at t.  Every path other than the best differs from it somewhere, so the
    second-best score is max over t and j != p*_t of mu_t[j].  Returns [B].
    """
    S0 = np.asarray(S0, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    B = S0.shape[0]
    L = S.shape[1] + 1
    alpha = np.zeros((B, L, K))
    beta = np.zeros((B, L, K))
    alpha[:, 0] = S0
    for t in range(1, L):
        alpha[:, t] = np.max(alpha[:, t - 1][:, :, None] + S[:, t - 1], axis=1)
    for t in range(L - 2, -1, -1):
        beta[:, t] = np.max(S[:, t] + beta[:, t + 1][:, None, :], axis=2)
    mu = alpha + beta
    best = np.max(mu[:, L - 1], axis=1)
    pstar = np.argmax(mu, axis=2)                    # best path's slot at each t
    masked = mu.copy()
    np.put_along_axis(masked, pstar[:, :, None], -np.inf, axis=2)
    second = np.max(masked.reshape(B, -1), axis=1)
    return best - second


# ------------------------------------------------------------------ f4 sampling
def sample_path(S0: np.ndarray, S: np.ndarray, top_idx: np.ndarray, T: float, u: np.ndarray):
    """The sampling walk ([POST] "A lightweight path selector": besides the
    greedy walk, sampling draws from the same precomputed scores; [GLONCE]
    lists a greedy choice, a draw, and a draw checked by rejection as the
    three ways the serial walk can end).

    Reading: the sampling twin of the greedy best-successor walk.  Starting
    from the last verified token, each position's slot is drawn from the
    temperature softmax of the scores of the successors of the slot drawn
    before:
      q_0 = softmax(S0 / T),  q_t = softmax(S[t-1, p_{t-1}, :] / T),
    p_t = the first slot j with u[b, t] < q_t[0] + ... + q_t[j] (inverse CDF
    with the given uniforms; if rounding leaves u above the last sum, the
    last slot with q > 0).  fp64 throughout.
    Returns (slot int32 [B, L], tok int32 [B, L], q fp64 [B, L, 16]): q[b, t]
    is the proposal distribution position t's token was drawn from.
    """
    S0 = np.asarray(S0, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    B = S0.shape[0]
    L = S.shape[1] + 1
    b = np.arange(B)
    slot = np.zeros((B, L), dtype=np.int64)
    q = np.zeros((B, L, K))
    for t in range(L):
        row = S0 if t == 0 else S[b, t - 1, slot[:, t - 1]]
        e = np.exp((row - row.max(axis=1, keepdims=True)) / T)
        q[:, t] = e / e.sum(axis=1, keepdims=True)
        cum = np.cumsum(q[:, t], axis=1)
        j = (u[:, t, None] >= cum).sum(axis=1)          # first j with u < cum_j
        last = K - 1 - np.argmax(q[:, t, ::-1] > 0, axis=1)
        slot[:, t] = np.minimum(j, last)
    tok = np.take_along_axis(np.asarray(top_idx), slot[:, :, None], axis=2)[:, :, 0]
    return slot.astype(np.int32), tok.astype(np.int32), q


def sample_path_joint(S0: np.ndarray, S: np.ndarray, top_idx: np.ndarray, T: float,
                      u: np.ndarray):
    """Sampling of a whole path from the same scores ([POST] "A lightweight
    path selector": sampling draws from the precomputed scores), the
    sampling twin of the max-plus walk: a slot path p is drawn with
    probability proportional to exp(score(p) / T), where
    score(p) = S0[p_0] + sum_t S[t-1, p_{t-1}, p_t].

    Reading: where the max-plus walk takes the best path, this draws from
    the distribution over all 16^L paths that the same scores define.  It is
    drawn by backward messages and forward draws (the same distribution as
    forward filtering and backward sampling; the forward order gives each
    position's proposal conditioned on the slots before it, which is what
    the rejection verification reads):
      beta_{L-1}[j] = 0,
      beta_t[i] = log sum_j exp(S[t, i, j] / T + beta_{t+1}[j])   (t = L-2 .. 0),
      q_0[j] proportional to exp(S0[j] / T + beta_0[j]),
      q_t[j] proportional to exp(S[t-1, p_{t-1}, j] / T + beta_t[j]),
    each p_t drawn by inverse CDF in slot order with u[b, t] (as in
    sample_path; if rounding leaves u above the last sum, the last slot with
    q > 0).  fp64 throughout.
    Returns (slot int32 [B, L], tok int32 [B, L], q fp64 [B, L, 16]): q[b, t]
    is the conditional proposal position t's token was drawn from.
    """
    S0 = np.asarray(S0, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    B = S0.shape[0]
    L = S.shape[1] + 1
    b = np.arange(B)

    def lse(a, axis):
        m = a.max(axis=axis, keepdims=True)
        return (m + np.log(np.exp(a - m).sum(axis=axis, keepdims=True))).squeeze(axis)

    beta = np.zeros((B, L, K))
    for t in range(L - 2, -1, -1):
        beta[:, t] = lse(S[:, t] / T + beta[:, t + 1][:, None, :], axis=2)
    slot = np.zeros((B, L), dtype=np.int64)
    q = np.zeros((B, L, K))
    for t in range(L):
        row = S0 if t == 0 else S[b, t - 1, slot[:, t - 1]]
        a = row / T + beta[:, t]
        e = np.exp(a - a.max(axis=1, keepdims=True))
        q[:, t] = e / e.sum(axis=1, keepdims=True)
        cum = np.cumsum(q[:, t], axis=1)
        j = (u[:, t, None] >= cum).sum(axis=1)          # first j with u < cum_j
        last = K - 1 - np.argmax(q[:, t, ::-1] > 0, axis=1)
        slot[:, t] = np.minimum(j, last)
    tok = np.take_along_axis(np.asarray(top_idx), slot[:, :, None], axis=2)[:, :, 0]
    return slot.astype(np.int32), tok.astype(np.int32), q


def sample_margin(q: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Distance of each uniform to the nearest boundary of its inverse-CDF
    bins (fp64, [B, L]): a perturbation of the probabilities smaller than
    this cannot change the drawn slot."""
    cum = np.concatenate([np.zeros(q.shape[:-1] + (1,)), np.cumsum(q, axis=-1)], axis=-1)
    return np.min(np.abs(cum - np.asarray(u, np.float64)[..., None]), axis=-1)


def target_lse(z_target: np.ndarray, T: float) -> np.ndarray:
    """log sum_v exp(z[v] / T) of every target row, fp64 ([..., V] -> [...])."""
    a = np.asarray(z_target, dtype=np.float64) / T
    m = a.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(a - m).sum(axis=-1, keepdims=True)))[..., 0]


def rejection_verify(path_tok: np.ndarray, q: np.ndarray, top_idx: np.ndarray,
                     z_target: np.ndarray, T: float, u_acc: np.ndarray, u_res: np.ndarray):
    """Lossless verification of a sampled path ([POST] "A lightweight path
    selector": the rejection step makes the emitted tokens follow the
    target's own distribution; [GLONCE] says the same of the final choice).

    The standard speculative-sampling rule (Leviathan et al. 2023; Chen et
    al. 2023).  The target's distribution at position t is
    p_t = softmax(z_target[b, t] / T) over the whole vocabulary (position L
    is the one after a fully accepted block); the proposal q_t is the
    16-candidate distribution the path's token was drawn from (zero off the
    candidates).  For t = 0, 1, ...: accept x_t when u_acc[b, t] * q_t(x_t) <
    p_t(x_t) (probability min(1, p/q)); at the first rejection n, the
    verifier's token is drawn from the residual max(0, p_n - q_n), normalised;
    if all L are accepted, it is drawn from p_L.  Draws use the inverse CDF
    in token-id order with u_res[b] scaled by the residual mass.  When
    rounding puts u_res * mass past the last partial sum, the draw takes the
    last token with mass; if no token has residual mass at all (possible only
    through rounding), the last token with p > 0; if none, the last token.
    Returns (accept_len int32 [B] = n + 1, next_tok int32 [B]).
    """
    path_tok = np.asarray(path_tok)
    top_idx = np.asarray(top_idx)
    B, L = path_tok.shape
    z = np.asarray(z_target, dtype=np.float64)
    lse = target_lse(z, T)                                  # [B, L+1]
    acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < L:
            x = path_tok[b, n]
            p_x = np.exp(z[b, n, x] / T - lse[b, n])
            q_x = q[b, n][top_idx[b, n] == x].sum()
            if u_acc[b, n] * q_x < p_x:
                n += 1
            else:
                break
        p = np.exp(z[b, n] / T - lse[b, n])
        if n < L:
            qv = np.zeros_like(p)
            np.add.at(qv, top_idx[b, n], q[b, n])
            r = np.maximum(p - qv, 0.0)
        else:
            r = p
        cum = np.cumsum(r)
        v = int(np.searchsorted(cum, u_res[b] * cum[-1], side="right"))
        if v >= len(r) or r[v] == 0.0:                       # rounding past the end
            nz = np.nonzero(r > 0)[0]
            if len(nz) == 0:                                 # no residual mass at all
                nz = np.nonzero(p > 0)[0]
            v = int(nz[-1]) if len(nz) else len(r) - 1
        acc[b], nxt[b] = n + 1, v
    return acc, nxt


# ------------------------------------------------------------------ a6 verify
def verify_greedy(path_tok: np.ndarray, target: np.ndarray):
    """Greedy verification and acceptance length ([POST] "The right token is
    already in the candidates", Table 1 caption: the acceptance length counts
    the verifier's next token).

    The target's argmax per position target [B, L+1] (target[:, L] is the
    verifier's token after a fully accepted block).  n = number of leading
    positions where the path equals the target; accept_len = n + 1 and the
    verifier contributes target[b, n].  Returns (accept_len, next_tok) int32 [B].
    """
    path_tok = np.asarray(path_tok)
    target = np.asarray(target)
    B, L = path_tok.shape
    match = path_tok == target[:, :L]
    n = np.cumprod(match, axis=1).sum(axis=1)
    return (n + 1).astype(np.int32), target[np.arange(B), n].astype(np.int32)


def oracle_selector(top_idx: np.ndarray, target: np.ndarray) -> np.ndarray:
    """The post's oracle selector ([POST] "The right token is already in the
    candidates"): at every position it picks the target's token whenever it is
    among the 16 candidates (else the top-1).  Returns path_tok [B, L]."""
    top_idx = np.asarray(top_idx)
    B, L, _ = top_idx.shape
    tgt = np.asarray(target)[:, :L]
    hit = (top_idx == tgt[:, :, None]).any(axis=2)
    return np.where(hit, tgt, top_idx[:, :, 0]).astype(np.int32)


def expected_acceptance(p) -> float:
    """Mean acceptance length when position t is right with probability p[t],
    given all earlier positions are right (Table 1's conditional recall):
    E = 1 + sum_k prod_{t <= k} p[t]  (the 1 is the verifier's token)."""
    return float(1.0 + np.sum(np.cumprod(np.asarray(p, dtype=np.float64))))


# ------------------------------------------------------------------ composition
def run_step_head(w, inp: Dict[str, object], y: np.ndarray,
                  blocks: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """logits -> top-16 -> [context gate] -> pair scores -> path, from the
    final hidden states y (fp64 values of the stored activations, [Bs, L, H])
    of the given blocks (all when None).  Returns every intermediate."""
    anchor_tok = inp["anchor_tok"]
    u_path = inp.get("u_path")
    if blocks is not None:
        anchor_tok = anchor_tok[blocks]
        u_path = None if u_path is None else u_path[blocks]
    Bs, L, H = y.shape
    z = lm_logits(y.reshape(Bs * L, H), inp["W"], w.dtype)
    top_val, top_idx = topk16(z)
    tv = top_val.reshape(Bs, L, K)
    ti = top_idx.reshape(Bs, L, K)
    gate = None
    if getattr(w, "gate", False):
        gate = context_gate(y.reshape(Bs * L, H), inp["Wg"], w.dtype).reshape(Bs, L, -1)
    S0, S = pair_scores(tv, ti, anchor_tok, inp["U"], inp["Vf"], w.dtype, gate)
    walk = getattr(w, "walk", "viterbi")
    q = score = None
    if walk == "sample":
        slot, tok, q = sample_path(S0, S, ti, w.temperature, u_path)
    elif walk == "sample-path":
        slot, tok, q = sample_path_joint(S0, S, ti, w.temperature, u_path)
    else:
        slot, tok, score = (path_select_greedy if walk == "greedy" else path_select)(S0, S, ti)
    return {"y": y, "z": z, "top_val": tv, "top_idx": ti, "gate": gate, "S0": S0, "S": S,
            "path_slot": slot, "path_tok": tok, "path_score": score, "q": q}


def run_step_front(w, inp: Dict[str, object], blocks: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """conv chain -> logits -> top-16 -> pair scores -> path, for the given
    blocks (all when None).  Verification needs targets and is run by the
    caller (verify_greedy, or rejection_verify for a sampled walk, whose
    proposal distributions come back as "q").  Returns every intermediate."""
    x = inp["x"]
    convs = inp["convs"]
    if blocks is not None:
        x = x[blocks]
        convs = [dict(c, anchor_h=c["anchor_h"][blocks]) for c in convs]
    xd = as_f64(x, w.dtype)
    cd = []
    for c in convs:
        if c.get("projT") is not None:          # [2G, H] storage -> [H, 2G] map
            proj = as_f64(c["projT"], w.dtype).T
        elif c["proj"] is not None:
            proj = np.asarray(c["proj"], np.float64)
        else:
            proj = None
        cd.append({"anchor_h": as_f64(c["anchor_h"], w.dtype),
                   "k0": np.asarray(c["k0"], np.float64), "k1": np.asarray(c["k1"], np.float64),
                   "proj": proj, "groups": c.get("groups", 1)})
    y = conv_chain(xd, cd, w.dtype)
    return run_step_head(w, inp, y, blocks)
