"""CPU oracle for the DFlash 2 draft-select-verify step -- TEST INFRASTRUCTURE.

This package is the plain, slow, obviously correct statement of what the
step computes.  It exists to check the HIP library, and only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it.  The product
path (``block_drafting_amd``) never imports, links or calls anything here,
and nothing here imports the product path.

Every function follows one passage of "DFlash 2: Keep Drafting Parallel"
(Inco AI's post) or the workload definitions, cited in its docstring.
Arithmetic is fp64 unless a step is defined in another precision (the path
walk decides in fp32, the precision of the kernel, so both sides take the
same argmax decisions).

Pins: every function is pinned against something other than itself in
``tests/test_oracle_pins.py`` (brute force, closed forms, invariants, the
pages' Table 1, special cases).  No function here is "parity unpinned".
"""
from .cpu_oracle import (  # noqa: F401
    as_f64,
    bf16_bits_to_f64,
    round_to_bf16,
    round_to_dtype,
    twotap_conv,
    conv_chain,
    lm_logits,
    canonical_logits,
    topk16,
    topk_gaps,
    pair_scores,
    context_gate,
    path_select,
    path_select_greedy,
    greedy_margin,
    path_scores_f64,
    path_margin,
    verify_greedy,
    sample_path,
    sample_path_joint,
    sample_margin,
    target_lse,
    rejection_verify,
    oracle_selector,
    expected_acceptance,
    run_step_front,
    run_step_head,
)
