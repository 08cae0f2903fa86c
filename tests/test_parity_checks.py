"""The parity checkers of the GPU tests, on the CPU with crafted logits: a wrong
greedy token must fail unless the oracle's own top-2 margin is within the tie bound
of the path's tolerance, and then only a near-tied candidate may be picked."""
import numpy as np
import pytest

from gpu_common import TIERS, check_close, check_tokens, tie_bound

F32, BF16 = TIERS["f32"], TIERS["bf16"]


def test_wrong_pick_with_large_margin_fails():
    # GPU [0, 0, 0, 10] against oracle [10, 0, 0, 0]: margin 10, far above any bound.
    with pytest.raises(AssertionError, match="picks 3, oracle 0"):
        check_tokens(np.array([[0.0, 0.0, 0.0, 10.0]]), np.array([[10.0, 0.0, 0.0, 0.0]]), BF16)


def test_equal_picks_pass_and_report_no_exemption():
    g = np.array([[0.1, 2.0, -1.0], [5.0, 4.9, 0.0]])
    toks, exempt = check_tokens(g, g + 1e-7, F32)
    assert toks == [1, 0] and exempt == []


def test_flip_inside_tie_bound_is_exempt_but_a_far_candidate_is_not():
    ref = np.array([[3.0, 3.0 - 1e-4, 0.0, 2.0]])
    tau = tie_bound(ref[0], BF16)
    assert 1e-4 < tau < 1.0
    toks, exempt = check_tokens(np.array([[3.0, 3.01, 0.0, 2.0]]), ref, BF16)  # picks the near-tied index 1
    assert toks == [1] and exempt == [0]
    with pytest.raises(AssertionError, match="beyond the tie bound"):      # picks index 3, 1.0 below the top
        check_tokens(np.array([[3.0, 2.9, 0.0, 3.5]]), ref, BF16)


def test_bound_is_fixed_by_the_tolerance_not_by_the_measured_error():
    # The same wrong pick fails however large the GPU's own error on that row is.
    ref = np.array([[1.0, 0.0, 0.5]])
    gpu = np.array([[1.0, 0.0, 100.0]])
    with pytest.raises(AssertionError):
        check_tokens(gpu, ref, F32)


def test_lowest_index_on_exact_ties():
    toks, _ = check_tokens(np.array([[2.0, 7.0, 7.0]]), np.array([[2.0, 7.0, 7.0]]), F32)
    assert toks == [1]


def test_f32_tier_rejects_a_convention_slip():
    # A slip of the size a lost rounding step or a wrong epsilon leaves (1e-4 on values
    # of order 1) passes the 2e-2 contract but not the fp32 tier.
    ref = np.linspace(-2, 2, 64)
    slipped = ref * (1 + 1e-4)
    check_close(slipped, ref, "contract")
    with pytest.raises(AssertionError, match="out of tolerance"):
        check_close(slipped, ref, "f32 tier", *F32)
