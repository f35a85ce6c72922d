"""Planted mistakes in the oracle must each fail at least one pin.

The oracle's C source carries ORACLE_PLANT_* switches; each build below turns
one on, and the pins of test_oracle_pins.py run against that build. A pin set
that let any of these through would not be pinning the oracle.
"""
import os

import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = ["DROP_SCALE", "DIVIDE_SCALE", "STRICT_MASK", "TOP_LEFT", "SWAP_KV", "TRANSPOSED_K",
           "NO_MAX", "NO_NORMALISE", "LOG2", "LSE_NO_MAX", "EMPTY_LSE_ZERO"]


def _pin_calls():
    calls = [(f"golden:{c['name']}", pins.test_handworked_golden, (c,)) for c in pins._golden_cases()]
    calls += [
        ("q_zero", pins.test_q_zero_gives_prefix_mean_of_v, (13, 5, True)),
        ("q_zero_cross", pins.test_q_zero_gives_prefix_mean_of_v, (5, 13, True)),
        ("single_key", pins.test_single_key_returns_v_exactly, (4,)),
        ("masked_rows", pins.test_fully_masked_rows_are_zero_even_with_nan_queries, ()),
        ("no_keys", pins.test_no_keys_at_all, ()),
        ("dominant", pins.test_dominant_key_selects_its_value, ()),
        ("brute", pins.test_brute_force_tiny_grid, (2, 3, 17, 33, 8, True)),
        ("brute_nc", pins.test_brute_force_tiny_grid, (1, 1, 5, 7, 4, False)),
        ("sdpa", pins.test_matches_torch_sdpa_float64, (2, 2, 96, 300, 128, True)),
        ("key_shift", pins.test_key_shift_invariance_at_overflow_scale, ()),
        ("beyond_exp", pins.test_scores_beyond_double_exp_range, ()),
        ("slicing", pins.test_bottom_right_slicing, (17,)),
    ]
    return calls


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistake_is_caught(mutant, tmp_path):
    path = oracle.build(force=True, out=str(tmp_path / f"liboracle_{mutant}.so"),
                        defines=[f"ORACLE_PLANT_{mutant}"])
    bad = oracle.load(path)
    saved = oracle._lib
    caught = []
    try:
        oracle._lib = bad
        for name, fn, args in _pin_calls():
            try:
                fn(*args)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(name)
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught planted mistake {mutant}"


def test_unplanted_build_passes_every_pin():
    for name, fn, args in _pin_calls():
        fn(*args)
