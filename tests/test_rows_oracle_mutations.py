"""Planted mistakes in the row-softmax oracle must each fail at least one pin.

rows_oracle.c carries ROWS_PLANT_* switches; each build below turns one on and
runs the pins of test_rows_oracle_pins.py against it.
"""
import pytest

import oracle
import test_rows_oracle_pins as pins

MUTANTS = ["NO_MAX", "MASK_IN_MAX", "TOP_LEFT", "LSE_LOG2", "EMPTY_UNIFORM", "BWD_NO_DOT", "BWD_SIGN"]


def _pin_calls():
    return [
        ("constant", pins.test_constant_row_is_uniform_and_lse_is_c_plus_log_n, (7,)),
        ("logistic", pins.test_two_entry_rows_are_logistic, ()),
        ("scipy", pins.test_matches_scipy_softmax_and_logsumexp, (17, 333)),
        ("shift", pins.test_shift_far_beyond_exp_range, ()),
        ("blocked", pins.test_masked_blocked_entries_never_reach_the_arithmetic, ()),
        ("one_hot", pins.test_masked_single_admitted_entry_is_one_hot, ()),
        ("empty", pins.test_rows_admitting_nothing_are_zero, ()),
        ("causal", pins.test_scaled_causal_matches_scipy_on_the_admitted_prefix, (20, 7, True, 0.125)),
        ("causal_wide", pins.test_scaled_causal_matches_scipy_on_the_admitted_prefix, (7, 20, True, 1.0)),
        ("bwd_fd", pins.test_softmax_backward_matches_finite_differences, (0.25,)),
        ("bwd_torch", pins.test_softmax_backward_matches_torch_float64_autograd, ()),
        ("bwd_closed", pins.test_softmax_backward_closed_forms, ()),
    ]


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistake_is_caught(mutant, tmp_path):
    path = oracle.build(force=True, out=str(tmp_path / f"liboracle_rows_{mutant}.so"),
                        defines=[f"ROWS_PLANT_{mutant}"])
    bad = oracle.load(path)
    saved = oracle._lib
    caught = []
    try:
        oracle._lib = bad
        for name, fn, args in _pin_calls():
            try:
                with __import__("numpy").errstate(all="ignore"):
                    fn(*args)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(name)
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught planted mistake {mutant}"


def test_unplanted_build_passes_every_pin():
    for name, fn, args in _pin_calls():
        fn(*args)
