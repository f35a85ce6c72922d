"""Planted mistakes in the masked attention oracle must each fail at least one pin.

attention_masked_oracle.c carries MASK_PLANT_* switches; each build below turns one on and
runs the pins of test_masked_oracle_pins.py against it.
"""
import numpy as np
import pytest

import oracle
import test_masked_oracle_pins as pins

MUTANTS = ["INVERT", "IGNORE_CAUSAL", "NO_MAX"]


def _pin_calls():
    return [
        ("scipy", pins.test_matches_scipy_on_the_admitted_entries, (0.5, True)),
        ("causal", pins.test_causal_pattern_as_a_mask_equals_the_causal_flag, (5, 11)),
        ("single", pins.test_single_admitted_key_returns_its_value_row, ()),
        ("and", pins.test_mask_and_causal_combine_by_and, ()),
        ("shift", pins.test_scores_beyond_the_exp_range, ()),
    ]


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistake_is_caught(mutant, tmp_path):
    path = oracle.build(force=True, out=str(tmp_path / f"liboracle_mask_{mutant}.so"),
                        defines=[f"MASK_PLANT_{mutant}"])
    bad = oracle.load(path)
    saved = oracle._lib
    caught = []
    try:
        oracle._lib = bad
        for name, fn, args in _pin_calls():
            try:
                with np.errstate(all="ignore"):
                    fn(*args)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(name)
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught planted mistake {mutant}"


def test_unplanted_build_passes_every_pin():
    for name, fn, args in _pin_calls():
        fn(*args)
