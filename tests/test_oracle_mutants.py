"""The oracle's pins are sharp: each test plants one plausible mistake in an
oracle function (on the CPU, through monkeypatch, for the duration of the
test only) and checks that a pin in test_oracle_pins.py then fails.  A pin
that still passed with the mistake planted would not be pinning that part of
the function."""
import numpy as np
import pytest

import oracle as O
import test_oracle_pins as pins


def _fails(*pin_calls):
    for call in pin_calls:
        with pytest.raises(AssertionError):
            call()


# ------------------------------------------------------------------ bf16 rounding
def test_pins_catch_truncating_bf16_rounding(monkeypatch):
    def truncate(v):
        f = np.asarray(v, dtype=np.float64).astype(np.float32)
        return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)

    monkeypatch.setattr(O, "round_to_bf16", truncate)
    _fails(pins.test_bf16_round_matches_torch_cast_on_f32_values,
           pins.test_bf16_round_ties_to_even_and_rounds_once)


def test_pins_catch_double_rounding_through_fp32(monkeypatch):
    orig = O.round_to_bf16
    monkeypatch.setattr(O, "round_to_bf16",
                        lambda v: orig(np.asarray(v, dtype=np.float64).astype(np.float32)
                                       .astype(np.float64)))
    _fails(pins.test_bf16_round_ties_to_even_and_rounds_once)


# ------------------------------------------------------------------ conv
def test_pins_catch_swapped_conv_taps(monkeypatch):
    orig = O.twotap_conv
    monkeypatch.setattr(O, "twotap_conv",
                        lambda x, a, k0, k1, *r, **kw: orig(x, a, k1, k0, *r, **kw))
    _fails(pins.test_conv_identity_taps_return_input_exactly,
           pins.test_conv_shift_taps_read_predecessor_and_anchor)


def test_pins_catch_a_dropped_anchor(monkeypatch):
    orig = O.twotap_conv
    monkeypatch.setattr(O, "twotap_conv",
                        lambda x, a, k0, k1, *r, **kw: orig(x, None, k0, k1, *r, **kw))
    _fails(pins.test_conv_shift_taps_read_predecessor_and_anchor)


def test_pins_catch_a_wrong_channel_to_group_map(monkeypatch):
    orig = O.twotap_conv

    def strided_groups(x, a, k0, k1, P=None, G=1):
        # channel c in group c % G instead of c // (H / G)
        if P is None or G == 1:
            return orig(x, a, k0, k1, P, G)
        B, L, H = x.shape
        first = np.zeros((B, 1, H)) if a is None else np.asarray(a, dtype=np.float64)[:, None]
        prev = np.concatenate([first, x[:, :-1]], axis=1)
        D = x @ P
        grp = np.arange(H) % G
        return (k0 + D[..., 2 * grp]) * x + (k1 + D[..., 2 * grp + 1]) * prev

    monkeypatch.setattr(O, "twotap_conv", strided_groups)
    _fails(pins.test_conv_one_hot_rows_recover_taps_and_corrections,
           pins.test_conv_per_16_channel_groups_reduce_to_one_group)


# ------------------------------------------------------------------ logits
def test_pins_catch_fp32_accumulation_of_the_logits(monkeypatch):
    def fp32_sums(y, W, w_dtype, chunk_elems=None):
        Wd = O.as_f64(W, w_dtype)
        return (np.asarray(y, np.float32) @ Wd.astype(np.float32).T).astype(np.float64)

    monkeypatch.setattr(O, "lm_logits", fp32_sums)
    _fails(pins.test_logits_are_exact_sums_rounded_once)


def test_pins_catch_a_transposed_weight_read(monkeypatch):
    orig = O.lm_logits

    def reversed_rows(y, W, w_dtype, *a, **kw):
        return orig(y, np.ascontiguousarray(np.asarray(W)[::-1]), w_dtype, *a, **kw)

    monkeypatch.setattr(O, "lm_logits", reversed_rows)
    _fails(pins.test_logits_one_hot_rows_return_weight_columns)


# ------------------------------------------------------------------ top-16
def test_pins_catch_ties_broken_by_the_higher_id(monkeypatch):
    def topk_high_id_first(z):
        z = np.asarray(z, dtype=np.float32)
        zc = np.where(np.isnan(z), -np.inf, z) + np.float32(0.0)   # -0 -> +0
        M, V = z.shape
        ids = np.arange(V)
        ti = np.stack([np.lexsort((-ids, -zc[m]))[:16] for m in range(M)]).astype(np.int32)
        return np.take_along_axis(zc, ti, axis=1), ti

    monkeypatch.setattr(O, "topk16", topk_high_id_first)
    _fails(lambda: pins.test_topk_matches_rank_counting_with_ties_zeros_nan_inf(0))


# ------------------------------------------------------------------ pair scores and gate
def test_pins_catch_swapped_pair_factors(monkeypatch):
    orig = O.pair_scores
    monkeypatch.setattr(O, "pair_scores",
                        lambda tv, ti, at, U, Vf, *r, **kw: orig(tv, ti, at, Vf, U, *r, **kw))
    _fails(pins.test_pair_scores_one_hot_factors_give_indicator_matches)


def test_pins_catch_a_dropped_anchor_match(monkeypatch):
    orig = O.pair_scores
    monkeypatch.setattr(O, "pair_scores",
                        lambda tv, ti, at, U, Vf, *r, **kw: orig(tv, ti, None, U, Vf, *r, **kw))
    _fails(pins.test_pair_scores_one_hot_factors_give_indicator_matches)


def test_pins_catch_the_previous_positions_gate(monkeypatch):
    orig = O.pair_scores

    def lagged_gate(tv, ti, at, U, Vf, dt, gate=None):
        return orig(tv, ti, at, U, Vf, dt, None if gate is None else np.roll(gate, 1, axis=1))

    monkeypatch.setattr(O, "pair_scores", lagged_gate)
    _fails(pins.test_gated_pair_scores_reduce_and_use_the_current_positions_gate)


def test_pins_catch_a_permuted_gate_map(monkeypatch):
    orig = O.context_gate
    monkeypatch.setattr(O, "context_gate",
                        lambda y, Wg, wd: orig(y, np.ascontiguousarray(np.asarray(Wg)[::-1]), wd))
    _fails(pins.test_context_gate_hand_values_and_orientation)


def test_pins_catch_a_missing_sigmoid(monkeypatch):
    def linear_gate(y, Wg, wd):
        return (np.asarray(y, np.float64) @ O.as_f64(Wg, wd).T).astype(np.float32)

    monkeypatch.setattr(O, "context_gate", linear_gate)
    _fails(pins.test_context_gate_hand_values_and_orientation,
           pins.test_context_gate_symmetry_and_library_logistic)


# ------------------------------------------------------------------ walks
def test_pins_catch_the_highest_slot_winning_ties(monkeypatch):
    orig = O.path_select

    def high_slot(S0, S, ti):
        slot, tok, score = orig(np.ascontiguousarray(S0[:, ::-1]),
                                np.ascontiguousarray(S[:, :, ::-1, ::-1]),
                                np.ascontiguousarray(ti[:, :, ::-1]))
        return 15 - slot, tok, score

    monkeypatch.setattr(O, "path_select", high_slot)
    _fails(*[lambda L=L, s=s: pins.test_path_select_matches_brute_force_on_dyadic_scores_with_ties(L, s)
             for L, s in ((2, 1), (3, 2))])


def test_pins_catch_transposed_pair_scores_in_the_walks(monkeypatch):
    ps, pg = O.path_select, O.path_select_greedy
    monkeypatch.setattr(O, "path_select",
                        lambda S0, S, ti: ps(S0, np.ascontiguousarray(S.transpose(0, 1, 3, 2)), ti))
    monkeypatch.setattr(O, "path_select_greedy",
                        lambda S0, S, ti: pg(S0, np.ascontiguousarray(S.transpose(0, 1, 3, 2)), ti))
    _fails(lambda: pins.test_path_select_matches_brute_force_on_continuous_scores(3, 6),
           pins.test_greedy_walk_hand_trap_differs_from_viterbi)


def test_pins_catch_a_sampling_walk_that_ignores_the_temperature(monkeypatch):
    orig = O.sample_path
    monkeypatch.setattr(O, "sample_path", lambda S0, S, ti, T, u: orig(S0, S, ti, 1.0, u))
    _fails(pins.test_sample_path_inverse_cdf_hand_case)


# ------------------------------------------------------------------ verification
def test_pins_catch_an_accept_test_without_the_uniform(monkeypatch):
    orig = O.rejection_verify
    monkeypatch.setattr(O, "rejection_verify",
                        lambda tok, q, top, z, T, ua, ur: orig(tok, q, top, z, T, ua * 0.0, ur))
    _fails(pins.test_rejection_verify_preserves_the_target_distribution)


def test_pins_catch_an_acceptance_without_the_verifiers_token(monkeypatch):
    orig = O.verify_greedy

    def no_bonus(path, tgt):
        acc, nxt = orig(path, tgt)
        return acc - 1, nxt

    monkeypatch.setattr(O, "verify_greedy", no_bonus)
    _fails(pins.test_verify_hand_cases, pins.test_verify_invariants_random)


def test_pins_catch_unconditional_recall_in_the_closed_form(monkeypatch):
    # treating Table 1's recall as independent per position: 1 + sum p_t
    monkeypatch.setattr(O, "expected_acceptance",
                        lambda p: float(1.0 + np.sum(np.asarray(p, dtype=np.float64))))
    _fails(pins.test_table1_acceptance_follows_from_recall_rows)


# ------------------------------------------------------------------ more planted mistakes
def test_pins_catch_a_chain_rounded_only_at_the_end(monkeypatch):
    def round_once(x, convs, dtype):
        y = np.asarray(x, dtype=np.float64)
        for c in convs:
            y = O.twotap_conv(y, c["anchor_h"], c["k0"], c["k1"], c.get("proj"),
                              c.get("groups", 1))
        return O.round_to_dtype(y, dtype)

    monkeypatch.setattr(O, "conv_chain", round_once)
    _fails(pins.test_conv_chain_rounds_each_application_to_storage_type)


def test_pins_catch_greedy_ties_to_the_highest_slot(monkeypatch):
    orig = O.path_select_greedy

    def high_slot(S0, S, ti):
        slot, tok, score = orig(np.ascontiguousarray(S0[:, ::-1]),
                                np.ascontiguousarray(S[:, :, ::-1, ::-1]),
                                np.ascontiguousarray(ti[:, :, ::-1]))
        return 15 - slot, tok, score

    monkeypatch.setattr(O, "path_select_greedy", high_slot)
    _fails(pins.test_greedy_walk_is_never_better_than_the_best_path)


def test_pins_catch_a_greedy_walk_from_the_wrong_row(monkeypatch):
    # the next row taken from the slot's position in the candidate list of
    # the wrong step: scores of step t read with step t+1's row index
    orig = O.path_select_greedy

    def shifted_rows(S0, S, ti):
        return orig(S0, np.ascontiguousarray(np.roll(S, 1, axis=1)), ti)

    monkeypatch.setattr(O, "path_select_greedy", shifted_rows)
    _fails(pins.test_greedy_walk_hand_trap_differs_from_viterbi)


def test_pins_catch_sampling_from_the_transposed_row(monkeypatch):
    orig = O.sample_path
    monkeypatch.setattr(O, "sample_path",
                        lambda S0, S, ti, T, u: orig(S0, np.ascontiguousarray(
                            np.swapaxes(S, -1, -2)), ti, T, u))
    _fails(pins.test_sample_path_inverse_cdf_hand_case,
           pins.test_sample_path_frequencies_and_low_temperature_limit)


def test_pins_catch_an_unshifted_log_sum_exp(monkeypatch):
    def unshifted(z, T):
        with np.errstate(over="ignore"):
            return np.log(np.exp(np.asarray(z, np.float64) / T).sum(axis=-1))

    monkeypatch.setattr(O, "target_lse", unshifted)
    _fails(pins.test_target_lse_matches_scipy_logsumexp)


def test_pins_catch_a_log_sum_exp_without_the_temperature(monkeypatch):
    orig = O.target_lse
    monkeypatch.setattr(O, "target_lse", lambda z, T: orig(z, 1.0))
    _fails(pins.test_target_lse_matches_scipy_logsumexp)


def test_pins_catch_sampling_margins_without_the_first_edge(monkeypatch):
    def upper_edges_only(q, u):
        cum = np.cumsum(q, axis=-1)
        return np.min(np.abs(cum - np.asarray(u, np.float64)[..., None]), axis=-1)

    monkeypatch.setattr(O, "sample_margin", upper_edges_only)
    _fails(pins.test_sample_margin_hand_case)


def test_pins_catch_top16_gaps_measured_on_one_side(monkeypatch):
    orig = O.topk_gaps

    def above_only(z, top_val):
        g = orig(z, top_val)
        vals = top_val.astype(np.float64)
        up = np.concatenate([np.full((g.shape[0], 1), np.inf), vals[:, :-1] - vals[:, 1:]], axis=1)
        return up

    monkeypatch.setattr(O, "topk_gaps", above_only)
    _fails(pins.test_topk_gaps)


def test_pins_catch_a_margin_between_final_states(monkeypatch):
    # the gap between the two best final slots of the max-plus recursion,
    # taken for the gap to the second best path (which may end in the same slot)
    def final_state_gap(S0, S):
        d = np.asarray(S0, np.float64)
        for t in range(S.shape[1]):
            d = (d[:, :, None] + np.asarray(S[:, t], np.float64)).max(axis=1)
        srt = -np.sort(-d, axis=1)
        return srt[:, 0] - srt[:, 1]

    monkeypatch.setattr(O, "path_margin", final_state_gap)
    _fails(pins.test_path_margin_when_the_second_path_shares_the_final_slot)


def test_pins_catch_the_largest_instead_of_the_smallest_greedy_gap(monkeypatch):
    def largest_gap(S0, S, slot):
        S0 = np.asarray(S0, np.float64)
        S = np.asarray(S, np.float64)
        B, L = slot.shape
        b = np.arange(B)
        gap = lambda row: (lambda s: s[:, 0] - s[:, 1])(-np.sort(-row, axis=1))
        m = gap(S0)
        for t in range(1, L):
            m = np.maximum(m, gap(S[b, t - 1, slot[:, t - 1]]))
        return m

    monkeypatch.setattr(O, "greedy_margin", largest_gap)
    _fails(pins.test_greedy_walk_hand_trap_differs_from_viterbi)


def test_pins_catch_a_residual_draw_from_p(monkeypatch):
    # at a rejection, drawing from p instead of max(0, p - q): the verifier
    # would re-propose the rejected candidates
    orig = O.rejection_verify

    def no_residual(path_tok, q, top_idx, z, T, u_acc, u_res):
        acc, nxt = orig(path_tok, q, top_idx, z, T, u_acc, u_res)
        zz = np.asarray(z, np.float64)
        lse = O.target_lse(zz, T)
        for b in range(len(acc)):
            n = acc[b] - 1
            p = np.exp(zz[b, n] / T - lse[b, n])
            cum = np.cumsum(p)
            v = int(np.searchsorted(cum, u_res[b] * cum[-1], side="right"))
            nxt[b] = min(v, len(p) - 1)
        return acc, nxt

    monkeypatch.setattr(O, "rejection_verify", no_residual)
    _fails(pins.test_rejection_verify_preserves_the_target_distribution)


def test_pins_catch_an_overshoot_that_takes_the_last_token(monkeypatch):
    # u * mass past the last partial sum answered with the row's last token,
    # whatever its mass (the GPU draw once did the same with its last tile)
    orig = O.rejection_verify

    def last_token(path_tok, q, top_idx, z, T, u_acc, u_res):
        acc, nxt = orig(path_tok, q, top_idx, z, T, u_acc, u_res)
        for b in range(len(acc)):
            if u_res[b] >= np.nextafter(1.0, 0.0):
                nxt[b] = np.asarray(z).shape[-1] - 1
        return acc, nxt

    monkeypatch.setattr(O, "rejection_verify", last_token)
    _fails(pins.test_rejection_verify_draw_edges)


def test_pins_catch_the_previous_token_taken_from_the_same_position(monkeypatch):
    orig = O.pair_scores

    def same_position(tv, ti, at, U, Vf, dt, gate=None):
        S0, S = orig(tv, ti, at, U, Vf, dt, gate)
        Ud, Vd = O.as_f64(U, dt), O.as_f64(Vf, dt)
        ti = np.asarray(ti)
        # S[t-1, i, j] with the previous factors of position t's candidates
        prev = Ud[ti[:, 1:]]
        cur = Vd[ti[:, 1:]]
        if gate is not None:
            prev = prev * np.asarray(gate, np.float64)[:, 1:, None, :]
        S = (np.asarray(tv, np.float64)[:, 1:, None, :] +
             np.einsum("btik,btjk->btij", prev, cur)).astype(np.float32)
        return S0, S

    monkeypatch.setattr(O, "pair_scores", same_position)
    _fails(pins.test_pair_scores_one_hot_factors_give_indicator_matches)


def test_pins_catch_scores_with_the_candidates_logit_of_the_wrong_slot(monkeypatch):
    # the unary term of the previous candidate i instead of the current j
    orig = O.pair_scores

    def row_unary(tv, ti, at, U, Vf, dt, gate=None):
        S0, S = orig(tv, ti, at, U, Vf, dt, gate)
        tvd = np.asarray(tv, np.float64)
        S = (S.astype(np.float64) - tvd[:, 1:, None, :] + tvd[:, 1:, :, None]).astype(np.float32)
        return S0, S

    monkeypatch.setattr(O, "pair_scores", row_unary)
    _fails(pins.test_pair_scores_zero_factors_reduce_to_unary,
           pins.test_pair_scores_one_hot_factors_give_indicator_matches)


# ------------------------------------------------------------------ whole-path sampling
def _joint_mutant(mistake):
    """sample_path_joint with one planted mistake in the backward messages or
    in the forward draws that read them."""
    def f(S0, S, top_idx, T, u):
        S0 = np.asarray(S0, np.float64)
        S = np.asarray(S, np.float64)
        u = np.asarray(u, np.float64)
        B, L = S0.shape[0], S.shape[1] + 1
        b = np.arange(B)
        beta = np.zeros((B, L + 1, 16))
        for t in range(L - 2, -1, -1):
            St = S[:, t].transpose(0, 2, 1) if mistake == "transposed" else S[:, t]
            a = St / T + beta[:, t + 1][:, None, :]
            m = a.max(axis=2)
            if mistake == "max":
                beta[:, t] = m
            elif mistake != "none":
                beta[:, t] = m + np.log(np.exp(a - m[:, :, None]).sum(axis=2))
        slot = np.zeros((B, L), np.int64)
        q = np.zeros((B, L, 16))
        for t in range(L):
            row = S0 if t == 0 else S[b, t - 1, slot[:, t - 1]]
            bt = beta[:, t + 1] if mistake == "next" else beta[:, t]
            a = row / T + bt
            e = np.exp(a - a.max(axis=1, keepdims=True))
            q[:, t] = e / e.sum(axis=1, keepdims=True)
            slot[:, t] = np.minimum((u[:, t, None] >= np.cumsum(q[:, t], axis=1)).sum(axis=1), 15)
        tok = np.take_along_axis(np.asarray(top_idx), slot[:, :, None], axis=2)[:, :, 0]
        return slot.astype(np.int32), tok.astype(np.int32), q
    return f


@pytest.mark.parametrize("mistake", ["none", "max", "transposed", "next"])
def test_pins_catch_mistakes_in_the_whole_path_sampler(monkeypatch, mistake):
    # none: no backward messages (the chain sampler); max: messages by max
    # instead of log-sum-exp; transposed: the recursion reads S[t, j, i];
    # next: position t's draw reads the message of position t + 1
    monkeypatch.setattr(O, "sample_path_joint", _joint_mutant(mistake))
    _fails(lambda: pins.test_joint_sampler_draws_the_path_distribution(3, 1.0),
           pins.test_joint_sampler_proposals_are_the_exact_conditionals)
